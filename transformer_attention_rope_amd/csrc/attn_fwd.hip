// Prefill attention forward for gfx950: GQA, causal sliding-window band,
// softmax, bf16 MFMA; q is rotated and normalised in the kernel, k arrives
// rotated and normalised from the input stage (attn_prep_kernel). Without a
// (cos, sin) table (nc_attn_fwd_normed) q arrives rotated and normalised too
// and the kernel only scales it.
//
// What is computed ("从文本到聊天模型" (onehacker.top) §5.4 score = Q K^T,
// softmax, weighted sum of V; §5.5 causal mask; §5.6 RoPE;
// "Nanochat与nanoGPT对比：关键升级" (lzwjava.github.io) §1 table and notes:
// QK-norm after RoPE, GQA, sliding window):
//   o[b,t,h] = sum_j P[t,j] v[b,j,g],  g = h / (H/Hkv),
//   P[t,:]   = softmax_j( q'[t].k'[j] / sqrt(D) ) over 0 <= kofs + t - j < W,
//   q', k'   = RMSNorm(RoPE(q)), RMSNorm(RoPE(k)) at positions pos_offset + t.
// kofs = 0 for the forward of a whole sequence; for a chunk prefilled into a
// cache (same page, §10.4) the queries are the chunk's, at key rows kofs ..,
// and the keys are the cache's rows 0 .. kofs + T - 1 (Tk rows per sequence).
//
// Design (bf16 path):
//  * k' is formed once per key row by the input stage: every key tile is
//    visited by several query tiles, and a copy costs the tile loop far less
//    than re-rotating and re-normalising it on each visit.
//  * A workgroup owns 256 query columns: hpw query heads of one K/V group
//    times 256/hpw consecutive positions, so a K/V tile staged in LDS serves
//    every head of the group. It is 8 waves (two per SIMD) of one 32-column
//    block each: one wave's MFMAs run while the other waits. At D = 128 that
//    fits the 256 registers of a wave with a fragment look-ahead of 3 MFMAs
//    and without the log-sum-exp output (calls that ask for it run the
//    2-wave form below, whose waves own two 32-column blocks each and may
//    use the whole register file, VGPRs and AGPRs).
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
//  * Staging is double-buffered twice over: tile kt is computed from one LDS
//    buffer while tile kt+1, loaded into registers during tile kt-1, is
//    written to the other, and the loads of tile kt+2 go out at the start of
//    tile kt into the second register set.
//  * A tile whose keys every column of a wave sees runs a fixed instruction
//    order in which the exponentials and the staging of the next tile sit
//    between the MFMAs: a wave issues vector instructions while its own
//    MFMAs execute, so this work hides under the matrix pipe. Tiles crossing
//    a wave's band edge are masked in place; tiles outside it are skipped
//    (the wave only stages). Heaviest query tiles are dispatched first.
//  * A band of at most half the sequence runs a form of 128 columns, 4 waves
//    of one column block, with two workgroups per compute unit: two waves per
//    SIMD again, and one workgroup's loads at its start and stores at its end
//    overlap the other's tiles. At D = 128 a 2-wave form (two column blocks
//    per wave, one wave per SIMD) serves the calls that ask for the row
//    log-sum-exp.
//  * A launch too small to fill the device (a chunk at a large offset, a batch
//    of one) cuts each query tile's key tiles into slices run by separate
//    workgroups; each writes unnormalised fp32 rows and row sums, which the
//    fixed exponent scale above lets a second kernel add directly.
//
// fp32 path: exact fp32 arithmetic on the vector ALUs (one thread per query
// column), same band, same softmax without a running maximum.
#include "device_common.hpp"
#include "launch.hpp"

#include <type_traits>
#include <utility>

namespace nc {

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1, expanded at
// compile time (the loop bodies below are too large for the unroller).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}
template <int I>
using ic = std::integral_constant<int, I>;

struct FwdArgs {
  const void* q;
  const void* kp;      // k' = RMSNorm(RoPE(k)), layout and type of k
  const void* v;
  void* o;
  const void* tabq;    // [T][D/2] (cos, sin) of positions pos_offset + t: fp16 pairs
                       // packed in 32 bits (bf16 kernel), float2 (fp32 kernel)
  int B, T, H, Hkv, W;
  int kofs;      // key row (= position) of query row 0: 0, or the chunk's offset in a cache
  int Tk;        // key rows per sequence in kp and v: T, or the cache length
  int G;         // H / Hkv
  int hpw_log2;  // log2(query heads per workgroup)
  int ngroups;   // H / hpw
  int nqt;       // query tiles per (b, head group)
  int bp_log2;   // log2(positions per workgroup)
  float qscale;  // log2(e) / sqrt(D): folded into q'
  int nsplit;    // workgroups per query tile, each over a slice of its key tiles
  int rows;      // B * T * H: output rows
  float* part;   // nsplit > 1: per slice, unnormalised fp32 output rows [nsplit][rows][D],
                 // then their row sums [nsplit][rows]
  float* lse;    // optional: per output row, ln of the softmax denominator, fp32 (rows of o)
};

// =====================================================================
// bf16 MFMA kernel
// =====================================================================
template <int D, int NW_ = 4>
struct BfCfg {
  // waves per workgroup: 4 (one per SIMD), 2 (one per SIMD, two workgroups
  // per compute unit) or 8 (two per SIMD)
  static constexpr int NW = NW_;
  static constexpr int NT = 64 * NW;       // threads per workgroup
  // 32-column blocks per wave: one with two waves per SIMD (8 waves, or 4
  // waves with two workgroups per compute unit), two in the 2-wave form
  static constexpr int CB = (NW == 8 || NW == 4) ? 1 : 2;
  static constexpr int NC = 32 * CB * NW;  // query columns per workgroup: 256, or 128 with 2 waves
  static constexpr int BN = 64;            // keys per tile
  static constexpr int KS = D / 16;        // MFMA k-steps of K Q^T
  static constexpr int DB = D / 32;        // 32-row blocks of O^T
  static constexpr int RB = BN / 32;       // 32-key blocks per tile
  static constexpr int PS = BN / 16;       // MFMA k-steps of V^T P^T
  static constexpr int VLD = BN + 8;       // LDS row stride of V^T (bf16)
  static constexpr int CPR = D / 8;        // 16-byte chunks per q, o or V row
  static constexpr int KCP = BN * D * 2 / 1024;    // 1 KB copies per K tile (64*16 bytes each)
  static constexpr int NKD = (KCP + NW - 1) / NW;  // K copies per wave per tile
  static constexpr int KSW = 128 / D;      // K rows per 64-bank span (swizzle period)
  static constexpr int NMB = (BN / 4) * CPR;       // 4-key x 8-dim V micro-blocks per tile
  static constexpr int NVB = (NMB + NT - 1) / NT;  // V micro-blocks per thread
  static constexpr int QLD = D + 8;        // LDS row stride of staged q / o rows (bf16)
  static constexpr int KBUF = BN * D;      // bf16 elements per K buffer (swizzled rows)
  static constexpr int VBUF = D * VLD;     // bf16 elements per V^T buffer
  // A tile is NM MFMAs: the score MFMAs (rb, s, cb) for m < NSM, then the
  // P.V MFMAs (s2, db, cb). Fragment f (K fragments (rb, s) first, then V
  // fragments (s2, db)) feeds MFMAs f*CB .. f*CB + CB-1.
  static constexpr int NSM = RB * KS * CB;
  static constexpr int NPM = PS * DB * CB;
  static constexpr int NM = NSM + NPM;
  static constexpr int NKF = RB * KS;
  static constexpr int NF = NKF + PS * DB;
  static constexpr int QR = 32 * CB;       // q / o rows per wave
  // V register sets: two (tile kt+2 loads while tile kt+1 is transposed),
  // except at D = 128 with two waves per SIMD, or with two waves per
  // workgroup (two V micro-blocks per thread): there one set (tile kt+1
  // loads at the start of tile kt and is transposed at its end) keeps the
  // kernel within its registers without spills
  static constexpr int VS = D == 128 ? 1 : 2;
  static constexpr int NQL = QR * CPR / 64;  // 16-byte row chunks per lane for them
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
// V^T rows hold BN keys in 16-byte chunks; chunk c of row d is stored at
// chunk position c ^ ((d >> 4) & 7). The transposing writes come from lanes
// whose rows are 8 apart, the fragment reads from lanes with consecutive
// rows: with a 72-element row stride and this swizzle both spread over all
// LDS banks.
__device__ __forceinline__ int vt_swz(int d, int col) {
  return ((((col >> 3) ^ (d >> 4)) & 7) << 3) | (col & 7);
}

// Kinds of tiles with a fixed instruction order, for a wave whose columns
// are consecutive positions starting on a 32-key boundary (64 of them from
// a tile boundary with two column blocks; 32 from half H of a tile with one):
//   kFull  every key visible to every column;
//   kDiag  the tile holding the wave's own positions (causal diagonal): key
//          blocks after the column block's own are skipped, the block on the
//          diagonal is masked (key <= query);
//   kWin   the first tile of the window (keys q - W ..): key blocks before
//          the column block's own are skipped, the block on the diagonal is
//          masked (key > query - W).
// A 32-key block rb and a column block cb lie on the diagonal when rb == cb
// (two column blocks) or rb == H (one).
enum TileKind { kFull = 0, kDiag = 1, kWin = 2 };

// Instruction order of such a tile, as a list of MFMAs: the score MFMAs
// (rb, s, cb) of the present 32x32 blocks, then their P.V MFMAs (s2, db, cb).
// Before MFMA m the K/V fragments fl[m][..] are read from LDS (each about
// LAM MFMAs before its first use); after MFMA m come the vector-work entries
// v[m][..]. Each slice has a first half (id) and a second half (id + 1000)
// issued one MFMA later, so the instructions between two MFMAs never wait on
// each other (a wave issues in order; a stalled instruction would hold the
// next MFMA):
//   200+8(rb*CB+cb)+i   2^S of score registers 2i, 2i+1 of block (rb, cb);
//                then packing into the P operand (masked on kDiag/kWin
//                diagonal blocks) and the row-sum update
//   100+4vb+m    transposition of the next tile's V micro-block vb, dims
//                pair m; then its two V^T rows into LDS      (if STAGE)
// Slices start in that order, spread evenly over the MFMAs. An exponential
// starts two MFMAs after the last score MFMA of its block, and a P.V MFMA
// comes after the second halves of the four slices that build its P operand.
template <int D, int NW, int KIND, bool STAGE, int H>
struct TileSched {
  using C = BfCfg<D, NW>;
  // fragment look-ahead in MFMAs: 8 fragments either way
  // (3 at D = 128 with one column block: the 8-wave form fits 256 registers
  // only with so short a look-ahead)
  static constexpr int MAXS = 24, MAXL = 16, LAM = C::CB == 2 ? 16 : (D == 128 ? 3 : 6);
  static constexpr int diag(int cb) { return C::CB == 2 ? cb : H; }
  static constexpr bool present(int rb, int cb) {
    return !((KIND == kDiag && rb > diag(cb)) || (KIND == kWin && rb < diag(cb)));
  }
  short mt[C::NM], ma[C::NM], mb[C::NM], mc[C::NM], mf[C::NM];
  short fl[C::NM][MAXL];
  short v[C::NM][MAXS];
  int nm, nsm, ok, nslices;
  constexpr TileSched()
      : mt{}, ma{}, mb{}, mc{}, mf{}, fl{}, v{}, nm(0), nsm(0), ok(1), nslices(0) {
    for (int rb = 0; rb < C::RB; ++rb)
      for (int s = 0; s < C::KS; ++s)
        for (int cb = 0; cb < C::CB; ++cb)
          if (present(rb, cb)) {
            mt[nm] = 0; ma[nm] = (short)rb; mb[nm] = (short)s; mc[nm] = (short)cb;
            mf[nm] = (short)(rb * C::KS + s);
            ++nm;
          }
    nsm = nm;
    for (int s2 = 0; s2 < C::PS; ++s2)
      for (int db = 0; db < C::DB; ++db)
        for (int cb = 0; cb < C::CB; ++cb)
          if (present(s2 / 2, cb)) {
            mt[nm] = 1; ma[nm] = (short)s2; mb[nm] = (short)db; mc[nm] = (short)cb;
            mf[nm] = (short)(C::NKF + s2 * C::DB + db);
            ++nm;
          }
    for (int m = 0; m < C::NM; ++m) {
      for (int k = 0; k < MAXL; ++k) fl[m][k] = -1;
      for (int k = 0; k < MAXS; ++k) v[m][k] = -1;
    }
    int nfl[C::NM] = {};
    for (int f = 0; f < C::NF; ++f) {
      int first = -1;
      for (int m = 0; m < nm && first < 0; ++m)
        if (mf[m] == f) first = m;
      if (first < 0) continue;
      const int at = first > LAM ? first - LAM : 0;
      if (nfl[at] < MAXL) fl[at][nfl[at]++] = (short)f; else ok = 0;
    }
    int last[2][2] = {{-1, -1}, {-1, -1}};  // [rb][cb]
    for (int m = 0; m < nsm; ++m) last[ma[m]][mc[m]] = m;

    short q[160] = {};
    short early[160] = {};  // first slot that keeps the exponential off the MFMA's result latency
    short ready[160] = {};  // first slot after the block's last score MFMA (program order)
    short start[160] = {};
    bool done[160] = {};
    int nq = 0;
    for (int s2 = 0; s2 < C::PS; ++s2)
      for (int cb = 0; cb < C::CB; ++cb)
        if (present(s2 / 2, cb))
          for (int i = 4 * (s2 % 2); i < 4 * (s2 % 2) + 4; ++i) {
            const int rb = s2 / 2;
            early[nq] = (short)(last[rb][cb] + 2);
            ready[nq] = (short)last[rb][cb];
            q[nq++] = (short)(200 + 8 * (rb * C::CB + cb) + i);
          }
    if (STAGE)
      for (int vb = 0; vb < C::NVB; ++vb)
        for (int m = 0; m < 4; ++m) q[nq++] = (short)(100 + 4 * vb + m);
    nslices = nq;
    int cnt[C::NM] = {};
    auto put = [&](int m, int id) {
      if (cnt[m] < MAXS) v[m][cnt[m]++] = (short)id; else ok = 0;
    };
    const int per_slot = (nq + nm - 1) / nm;
    int head = 0;
    for (int m = 0; m < nm; ++m) {
      for (int x = 0; x < nq; ++x)
        if (done[x] && start[x] == m - 1) put(m, q[x] + 1000);
      int started = 0;
      auto begin = [&](int x) {
        put(m, q[x]);
        done[x] = true;
        start[x] = (short)m;
        ++started;
      };
      // both halves in this slot (the P operand is needed by the next MFMA)
      auto begin_both = [&](int x) {
        put(m, q[x]);
        put(m, q[x] + 1000);
        done[x] = true;
        start[x] = -100;
        ++started;
      };
      // The P operand of MFMA m+1 must be complete after slot m, and that of
      // MFMA m+2 after slot m+1. A slice starts only after its block's last
      // score MFMA in program order (slot >= ready).
      for (int ahead = 1; ahead <= 2; ++ahead) {
        if (m + ahead >= nm || mt[m + ahead] != 1) continue;
        const int s2 = ma[m + ahead], cb = mc[m + ahead], rb = s2 / 2;
        for (int i = 4 * (s2 % 2); i < 4 * (s2 % 2) + 4; ++i) {
          const short id = (short)(200 + 8 * (rb * C::CB + cb) + i);
          for (int x = 0; x < nq; ++x)
            if (q[x] == id && !done[x]) {
              for (int y = head; y <= x; ++y)
                if (!done[y]) {
                  if (ahead == 1) {
                    if (q[y] >= 200 && ready[y] > m) ok = 0;  // P.V follows its scores
                    begin_both(y);
                  } else if (q[y] < 200 || ready[y] <= m) {
                    begin(y);
                  }
                }
            }
        }
      }
      while (head < nq && done[head]) ++head;
      const bool lastm = m == nm - 1;
      while ((started < per_slot || lastm) && head < nq && early[head] <= m) {
        begin(head);
        while (head < nq && done[head]) ++head;
      }
      if (lastm)
        for (int x = 0; x < nq; ++x)
          if (done[x] && start[x] == m) put(m, q[x] + 1000);
    }
    for (int x = 0; x < nq; ++x)
      if (!done[x]) ok = 0;
    for (int x = 0; x < nq; ++x)
      if (q[x] >= 200)
        for (int mp = 0; mp < ready[x]; ++mp)
          for (int k = 0; k < MAXS; ++k)
            if (v[mp][k] == q[x]) ok = 0;
    for (int m = nsm; m < nm; ++m) {
      const int s2 = ma[m], cb = mc[m], rb = s2 / 2;
      for (int i = 4 * (s2 % 2); i < 4 * (s2 % 2) + 4; ++i) {
        const int id = 1000 + 200 + 8 * (rb * C::CB + cb) + i;
        bool seen = false;
        for (int mp = 0; mp < m; ++mp)
          for (int k = 0; k < MAXS; ++k)
            if (v[mp][k] == id) seen = true;
        if (!seen) ok = 0;
      }
    }
  }
};
template <int D, int NW, int KIND, bool STAGE, int H>
struct TileSchedTab {
  static constexpr TileSched<D, NW, KIND, STAGE, H> s{};
  static_assert(s.ok, "tile schedule");
};

// The bf16 kernel body. With SPLIT, each workgroup runs one of nsplit slices
// of its query tile's key tiles and writes unnormalised fp32 partial rows
// (attn_split_combine_kernel adds them up); without, it writes o itself.
// LSE: whether the epilogue writes the row log-sum-exp (kLseNone: never;
// kLseIfGiven: when p.lse is set). The 8-wave D = 128 body has no registers
// to spare for it (with the write it spills), so it is built without; forward
// calls that ask for the log-sum-exp at D = 128 run the 2-wave body.
enum { kLseNone = 0, kLseIfGiven = 1 };
template <int D, int NW, bool SPLIT, int LSE = kLseIfGiven>
__device__ __forceinline__ void attn_fwd_bf16_body(const FwdArgs& p) {
  using C = BfCfg<D, NW>;
  constexpr int CB = C::CB;
  // K and V^T double buffers. Before the first tile and after the last one
  // the V^T part (enlarged to fit) holds each wave's q rows and output rows
  // (QLD-element rows, QR per wave) on their way between row-major global
  // memory and the MFMA register layouts; the K part is only written by the
  // tile copies, so the first one can start at once.
  constexpr int kVpart = 2 * C::VBUF > NW * C::QR * C::QLD ? 2 * C::VBUF : NW * C::QR * C::QLD;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * C::KBUF + kVpart];
  uint16_t* const Ks = smem;
  uint16_t* const Vt = smem + 2 * C::KBUF;

  const uint16_t* __restrict__ qg = (const uint16_t*)p.q;
  uint16_t* __restrict__ og = (uint16_t*)p.o;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int n = lane & 31, hf = lane >> 5;

  // ---- work item: heaviest (latest) query tiles first; a query tile's
  // ---- key-tile slices next to each other
  const int per_split = p.B * p.ngroups;
  const int per_qt = SPLIT ? per_split * p.nsplit : per_split;
  const int qt = p.nqt - 1 - (int)blockIdx.x / per_qt;
  const int rem0 = (int)blockIdx.x % per_qt;
  const int split = SPLIT ? rem0 / per_split : 0;
  const int rem = rem0 - split * per_split;
  const int b = rem / p.ngroups, grp = rem - (rem / p.ngroups) * p.ngroups;
  const int hpw = 1 << p.hpw_log2;
  // Everything below works in positions (= key rows): query row t sits at
  // position kofs + t, and q and o rows are addressed by position - kofs.
  const int q_end = p.kofs + p.T;                   // one past the last query position
  const int q0 = (qt << p.bp_log2) + p.kofs;        // position of the tile's first query
  const int q_last = min(q0 + (1 << p.bp_log2), q_end) - 1;
  const long long qo_row0 = (long long)b * p.T - p.kofs;  // q/o row of position 0 in sequence b
  const int g = (grp * hpw) / p.G;

  // ---- key-tile range of the workgroup's band [max(0, q0 - W + 1), q_last]
  const int k_first = max(0, q0 - p.W + 1);
  int kt0 = k_first / C::BN, kt1 = q_last / C::BN;
  // slice `split` of nsplit near-equal slices of the range (possibly empty)
  if constexpr (SPLIT) {
    const int n = kt1 - kt0 + 1;
    kt1 = kt0 + ((split + 1) * n) / p.nsplit - 1;
    kt0 += (split * n) / p.nsplit;
  }
  // slice outputs, formed where they are written
  auto part_o = [&]() __attribute__((always_inline)) { return p.part + (size_t)split * p.rows * D; };
  auto part_l = [&]() __attribute__((always_inline)) {
    return p.part + (size_t)p.nsplit * p.rows * D + (size_t)split * p.rows;
  };
  if (SPLIT && kt1 < kt0) {
    // an empty slice contributes nothing: zero output rows and row sums
    for (int i = threadIdx.x; i < C::NC * (D / 4); i += C::NT) {
      const int col = i / (D / 4), c4 = i - (i / (D / 4)) * (D / 4);
      const int tq = q0 + (col >> p.hpw_log2);
      if (tq < q_end) {
        const size_t row = (size_t)(qo_row0 + tq) * p.H + grp * hpw + (col & (hpw - 1));
        st16(part_o() + row * D + 4 * c4, u32x4_t{0u, 0u, 0u, 0u});
        if (c4 == 0) part_l()[row] = 0.f;
      }
    }
    return;
  }

  // ---- staging: buffer resources whose ranges end at key row kofs + T
  // ---- (reads past it return zeros), per-thread byte offsets, per-tile bases
  const uint32_t row_bytes = (uint32_t)p.Hkv * D * 2;
  const size_t kv_base = ((size_t)b * p.Tk * p.Hkv + g) * D;
  const uint32_t kv_records = (uint32_t)(((size_t)q_end * p.Hkv - g) * D * 2);
  const char* vseq = (const char*)((const uint16_t*)p.v + kv_base);
  const char* kseq = (const char*)((const uint16_t*)p.kp + kv_base);
  // the K row that copy j of this wave's lane fills in a tile, and the chunk
  // of it: LDS row r holds chunk c of global row r at position
  // c ^ ((r / KSW) % CPR), so the row-strided fragment reads spread over all
  // banks while every copy still reads whole rows
  uint32_t k_voff[C::NKD];
#pragma unroll
  for (int j = 0; j < C::NKD; ++j) {
    const int slot = (wave * C::NKD + j) * 64 + lane;  // 16-byte slot in the tile
    const int r = slot / C::CPR, c = slot % C::CPR;
    k_voff[j] = (uint32_t)r * row_bytes + (uint32_t)((c ^ ((r / C::KSW) % C::CPR)) * 16);
  }
  // V micro-block mb: dims 8*(mb % CPR) .. +7 of the 4 keys of key group
  // vgp, so a wave's load of one key slot covers whole rows. Key groups are
  // taken in the order 0, 2, 1, 3 within each run of four, which (with the
  // V^T swizzle) keeps the transposing LDS writes free of bank conflicts.
  uint32_t v_voff[C::NVB];
  int v_lds[C::NVB];
  bool v_act[C::NVB];
#pragma unroll
  for (int j = 0; j < C::NVB; ++j) {
    const int mb = tid + C::NT * j;
    const int vd = mb % C::CPR, grp4 = mb / C::CPR;
    const int vgp = (grp4 & ~3) | ((grp4 & 1) << 1) | ((grp4 >> 1) & 1);
    v_act[j] = mb < C::NMB;
    v_voff[j] = v_act[j] ? (uint32_t)(4 * vgp) * row_bytes + vd * 16 : 0xF0000000u;
    v_lds[j] = (8 * vd) * C::VLD + vt_swz(8 * vd, vt_pos(4 * vgp));
  }

  u32x4_t vw[C::VS][C::NVB][4];
  // register set the tile of parity P loads into, the set it transposes from,
  // and how many tiles ahead it loads
  constexpr auto lset = [](int P) { return C::VS == 2 ? P : 0; };
  constexpr auto sset = [](int P) { return C::VS == 2 ? (P ^ 1) : 0; };
  constexpr int VAHEAD = C::VS;

  // V rows of tile kt into register set S. The resource is rebased on the
  // tile's first key: rows past token T (and only those) fall beyond
  // num_records and read as zero. Every wave issues the same 4*NVB loads for
  // every tile, so the count of loads in flight is the same on every path:
  // a tile past the workgroup's range (kt > kt1) gets an empty range, and a
  // lane without a micro-block an offset past any range; both read nothing.
  auto gload = [&](auto Sc, int kt) __attribute__((always_inline)) {
    constexpr int S = decltype(Sc)::value;
    const uint32_t so = (uint32_t)kt * C::BN * row_bytes;
    const uint32_t nk =
        __builtin_amdgcn_readfirstlane(kt <= kt1 && so < kv_records ? kv_records - so : 0u);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vseq + so, nk);
#pragma unroll
    for (int j = 0; j < C::NVB; ++j) {
#pragma unroll
      for (int r = 0; r < 4; ++r) vw[S][j][r] = bload16(rv, v_voff[j] + r * row_bytes, 0);
    }
  };
  // V micro-block j of set S, dims pair m: rows 2m, 2m+1 of its V^T block,
  // 4 consecutive (permuted) key slots each
  auto v_pair = [&](auto Sc, int j, int m, uint16_t* vb) __attribute__((always_inline)) {
    constexpr int S = decltype(Sc)::value;
    const uint32_t a0 = vw[S][j][0][m], a1 = vw[S][j][1][m], a2 = vw[S][j][2][m], a3 = vw[S][j][3][m];
    const u32x2_t lo = {lo_halves(a0, a1), lo_halves(a2, a3)};
    const u32x2_t hi = {hi_halves(a0, a1), hi_halves(a2, a3)};
    st8(vb + v_lds[j] + (2 * m) * C::VLD, lo);
    st8(vb + v_lds[j] + (2 * m + 1) * C::VLD, hi);
  };
  // k' tile kt into LDS K buffer buf: each wave makes NKD copies of 1 KB
  // (16 bytes per lane) straight from memory to LDS. The resource is rebased
  // on the tile's first key, so rows past token T read as zero; a tile past
  // the workgroup's range gets an empty range (it fills the free buffer with
  // zeros and reads nothing). The copies count as loads (vmcnt): a wait for
  // them precedes the barrier that publishes the buffer.
  auto kcopy = [&](int kt, int buf) __attribute__((always_inline)) {
    const uint32_t so = (uint32_t)kt * C::BN * row_bytes;
    const uint32_t nk =
        __builtin_amdgcn_readfirstlane(kt <= kt1 && so < kv_records ? kv_records - so : 0u);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kseq + so, nk);
#pragma unroll
    for (int j = 0; j < C::NKD; ++j) {
      const int f = wave * C::NKD + j;
      if (C::NKD * C::NW == C::KCP || f < C::KCP) lds_copy16(rk, Ks + buf * C::KBUF + f * 512, k_voff[j]);
    }
  };
  // V register set S into LDS buffer buf
  auto stage = [&](auto Sc, int buf) __attribute__((always_inline)) {
    constexpr int S = decltype(Sc)::value;
    uint16_t* vb = Vt + buf * C::VBUF;
#pragma unroll
    for (int j = 0; j < C::NVB; ++j)
      if (C::NVB * C::NT == C::NMB || v_act[j]) {
#pragma unroll
        for (int m = 0; m < 4; ++m) v_pair(Sc, j, m, vb);
      }
  };

  // ---- this lane's query columns, one per 32-column block
  int t[CB], h[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int col = wave * 32 * CB + cb * 32 + n;
    t[cb] = q0 + (col >> p.hpw_log2);
    h[cb] = grp * hpw + (col & (hpw - 1));
  }

  // ---- Q: the wave's QR q rows are read row-major (CPR lanes per row, so
  // ---- every load covers whole rows), rotated with the table, RMS-
  // ---- normalised (sum over the row's lanes), scaled by log2(e)/sqrt(D) and
  // ---- rounded to bf16 there, written to the wave's LDS rows, and read back
  // ---- as the MFMA B operand (lane-half hf holds dims 16s + 8hf .. +7). The
  // ---- first V tiles go out after the q rows (the first k' tile before).
  constexpr int RPI = 64 / C::CPR;  // q rows per load
  uint16_t* const qs = Vt + wave * C::QR * C::QLD;
  // row r of the wave: column wave*QR + r
  auto col_row = [&](int r, int& tr, int& hr) __attribute__((always_inline)) {
    const int col = wave * C::QR + r;
    tr = q0 + (col >> p.hpw_log2);
    hr = grp * hpw + (col & (hpw - 1));
  };
  const int qc = lane % C::CPR, qr0 = lane / C::CPR;
  kcopy(kt0, 0);
  bf16x8_t bq[CB][C::KS];
  {
    // all rows and their table entries (one 16-byte load each: four fp16
    // (cos, sin) pairs) in one round trip
    constexpr int NB = 1;
    constexpr int PB = C::NQL;
    const uint32_t* const tab = reinterpret_cast<const uint32_t*>(p.tabq);
#pragma unroll
    for (int bt = 0; bt < NB; ++bt) {
      u32x4_t qw[PB];
      u32x4_t tq[PB];
#pragma unroll
      for (int ii = 0; ii < PB; ++ii) {
        const int i = bt * PB + ii;
        int tr, hr;
        col_row(i * RPI + qr0, tr, hr);
        const int tc = tr < q_end ? tr : q_end - 1;
        qw[ii] = ld16(qg + ((size_t)(qo_row0 + tc) * p.H + hr) * D + qc * 8);
        // no table: q rows arrive rotated and normalised; (cos, sin) = (1, 0)
        tq[ii] = tab != nullptr ? ld16(tab + (size_t)(tc - p.kofs) * (D / 2) + qc * 4)
                                : u32x4_t{0x3C00u, 0x3C00u, 0x3C00u, 0x3C00u};
      }
      if (bt == 0) {
        gload(ic<0>{}, kt0);
        if constexpr (C::VS == 2) gload(ic<1>{}, kt0 + 1);
      }
#pragma unroll
      for (int ii = 0; ii < PB; ++ii) {
        const int i = bt * PB + ii;
        float x[8];
        float ss = 0.f;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const float xe = bf_lo(qw[ii][m]), xo = bf_hi(qw[ii][m]);
          const float c = h_lo(tq[ii][m]), sn = h_hi(tq[ii][m]);
          const float ye = xe * c - xo * sn, yo = xe * sn + xo * c;
          x[2 * m] = ye;
          x[2 * m + 1] = yo;
          ss += ye * ye + yo * yo;
        }
        ss = dpp_group_sum<C::CPR>(ss);
        const float sc = tab != nullptr ? p.qscale * rsq(ss * (1.0f / D) + kEps) : p.qscale;
        u32x4_t w;
#pragma unroll
        for (int m = 0; m < 4; ++m) w[m] = pack_bf2(x[2 * m] * sc, x[2 * m + 1] * sc);
        st16(qs + (i * RPI + qr0) * C::QLD + qc * 8, w);
      }
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int s = 0; s < C::KS; ++s)
        bq[cb][s] = *reinterpret_cast<const bf16x8_t*>(qs + (cb * 32 + n) * C::QLD + 16 * s + 8 * hf);
  }

  f32x16_t oacc[C::DB][CB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][cb][r] = 0.f;
  float lsum[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) lsum[cb] = 0.f;

  // Positions covered by this wave (its 32*CB columns): [tw0, tw1].
  const int tw0 = q0 + ((wave * 32 * CB) >> p.hpw_log2);
  const int tw1 = min(q0 + ((wave * 32 * CB + 32 * CB - 1) >> p.hpw_log2), q_end - 1);
  constexpr uint32_t kOnes = 0x3F803F80u;  // bf16 pair (1, 1)

  // K fragment (rb, s): row rb*32 + n, chunk 2s + hf, at its swizzled position
  const int k_lane = n * D;
  const int k_swz = (n / C::KSW) % C::CPR;
  auto kfrag = [&](const uint16_t* kb, int rb, int s) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x8_t*>(kb + rb * 32 * D + k_lane + (((2 * s + hf) ^ k_swz) << 3));
  };
  // V^T fragment (s2, db): row db*32 + n, logical chunk 2*s2 + hf, stored at
  // chunk (2*s2 + hf) ^ (2*db + n/16) (the swizzle of vt_swz)
  const int vt_lane = n * C::VLD + 8 * (hf ^ (n >> 4));
  auto vfrag = [&](const uint16_t* vb, int s2, int db) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x8_t*>(vb + vt_lane + db * 32 * C::VLD + 16 * ((s2 ^ db) & 3));
  };

  // Tile crossing the band edge for this wave: 32-key blocks the wave cannot
  // see are skipped, blocks it sees in part are masked in place.
  auto compute_edge = [&](int buf, int kt) __attribute__((always_inline)) {
    const uint16_t* kb = Ks + buf * C::KBUF;
    const uint16_t* vb = Vt + buf * C::VBUF;
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb) {
      const int kb0 = kt * C::BN + rb * 32;
      if (kb0 > tw1 || tw0 - (kb0 + 31) >= p.W) continue;
      f32x16_t sc[CB];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[cb][r] = 0.f;
#pragma unroll
      for (int s = 0; s < C::KS; ++s) {
        const bf16x8_t a = kfrag(kb, rb, s);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          sc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq[cb][s], sc[cb], 0, 0, 0);
      }
      const bool all = kb0 + 31 <= tw0 && tw1 - kb0 < p.W;
      if (!all) {
        // key of register r is kb0 + 8*(r/4) + 4*hf + r%4
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const int dl0 = t[cb] - kb0 - 4 * hf;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int dl = dl0 - (8 * (r >> 2) + (r & 3));
            sc[cb][r] = ((unsigned)dl < (unsigned)p.W) ? sc[cb][r] : -INFINITY;  // 2^-inf = 0
          }
        }
      }
      bf16x8_t pb[CB][2];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          u32x4_t w;
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            w[m] = pack_bf2(fast_exp2(sc[cb][8 * s2 + 2 * m]), fast_exp2(sc[cb][8 * s2 + 2 * m + 1]));
            lsum[cb] = dot2bf(w[m], kOnes, lsum[cb]);
          }
          pb[cb][s2] = __builtin_bit_cast(bf16x8_t, w);
        }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const bf16x8_t a = vfrag(vb, 2 * rb + s2, db);
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
            oacc[db][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[cb][s2], oacc[db][cb], 0, 0, 0);
        }
    }
  };

  // Diagonal-block masks of kDiag tiles: pair i of a score block holds keys
  // c(2i), c(2i+1) with c(r) = 8*(r/4) + r%4 + 4*hf against query n; a key is
  // at or before the query iff c(r) <= n - 4*hf. One bf16 half per key.
  // Formed where used (only diagonal and window tiles), so that no register
  // holds them across the tile loop.
  auto dmask = [&](int i) __attribute__((always_inline)) -> uint32_t {
    const int e = n - 4 * hf;
    const int c0 = 8 * ((2 * i) >> 2) + ((2 * i) & 3), c1 = 8 * ((2 * i + 1) >> 2) + ((2 * i + 1) & 3);
    return (c0 <= e ? 0x0000ffffu : 0u) | (c1 <= e ? 0xffff0000u : 0u);
  };

  // Tile kt of parity P (LDS buffers P) of kind KIND, in a fixed instruction
  // order (TileSched): the k' copy of tile kt+1 into K buffer P^1 (if STAGE)
  // and the V loads of tile kt+2 into register set P go out first, then the
  // MFMAs of the tile run with the softmax of its scores and (if STAGE) the
  // transposition of tile kt+1's V (register set P^1, loaded a tile ago)
  // into V^T buffer P^1 in between.
  auto tile_sched = [&](auto Kc, auto Sc, auto Pc, auto Hc, int kt) __attribute__((always_inline)) {
    constexpr int KIND = decltype(Kc)::value;
    constexpr bool STAGE = decltype(Sc)::value != 0;
    constexpr int P = decltype(Pc)::value;
    constexpr int HALF = decltype(Hc)::value;
    using SCH = TileSchedTab<D, NW, KIND, STAGE, HALF>;
    using TS = TileSched<D, NW, KIND, STAGE, HALF>;
    const uint16_t* kb = Ks + P * C::KBUF;
    const uint16_t* vb = Vt + P * C::VBUF;
    uint16_t* vbw = Vt + (P ^ 1) * C::VBUF;
    if (STAGE) {
      kcopy(kt + 1, P ^ 1);
      __builtin_amdgcn_sched_barrier(0);  // the copies go out before the V loads
      gload(ic<lset(P)>{}, kt + VAHEAD);
    }
    f32x16_t sacc[C::RB][CB];
    u32x4_t pbu[CB][C::PS];
    bf16x8_t fr[C::NF];
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[rb][cb][r] = 0.f;
    auto frag = [&](int f) __attribute__((always_inline)) -> bf16x8_t {
      if (f < C::NKF) return kfrag(kb, f / C::KS, f % C::KS);
      const int fv = f - C::NKF;
      return vfrag(vb, fv / C::DB, fv % C::DB);
    };
    float etmp[C::RB * CB * 8][2];
    uint32_t vtmp[C::NVB][4][4];
    auto slice = [&](auto idc) __attribute__((always_inline)) {
      constexpr int id0 = decltype(idc)::value;
      constexpr bool second = id0 >= 1000;
      constexpr int id = second ? id0 - 1000 : id0;
      if constexpr (id0 < 0) {
      } else if constexpr (id < 200) {
        constexpr int j = (id - 100) >> 2, m = (id - 100) & 3;
        if (!(C::NVB * C::NT == C::NMB || v_act[j])) return;
        if constexpr (!second) {
          constexpr int SS = sset(P);
          const uint32_t a0 = vw[SS][j][0][m], a1 = vw[SS][j][1][m];
          const uint32_t a2 = vw[SS][j][2][m], a3 = vw[SS][j][3][m];
          vtmp[j][m][0] = lo_halves(a0, a1);
          vtmp[j][m][1] = lo_halves(a2, a3);
          vtmp[j][m][2] = hi_halves(a0, a1);
          vtmp[j][m][3] = hi_halves(a2, a3);
#pragma unroll
          for (int x = 0; x < 4; ++x) pin(vtmp[j][m][x]);
        } else {
          st8(vbw + v_lds[j] + (2 * m) * C::VLD, u32x2_t{vtmp[j][m][0], vtmp[j][m][1]});
          st8(vbw + v_lds[j] + (2 * m + 1) * C::VLD, u32x2_t{vtmp[j][m][2], vtmp[j][m][3]});
        }
      } else {
        constexpr int idx = id - 200;
        constexpr int rb = idx / (8 * CB), cb = (idx / 8) % CB, i = idx % 8;
        if constexpr (!second) {
          etmp[idx][0] = fast_exp2(sacc[rb][cb][2 * i]);
          etmp[idx][1] = fast_exp2(sacc[rb][cb][2 * i + 1]);
          pin(etmp[idx][0]);
          pin(etmp[idx][1]);
        } else {
          uint32_t w = pack_bf2(etmp[idx][0], etmp[idx][1]);
          if constexpr (KIND == kDiag && rb == TS::diag(cb)) w &= dmask(i);
          if constexpr (KIND == kWin && rb == TS::diag(cb)) w &= ~dmask(i);
          lsum[cb] = dot2bf(w, kOnes, lsum[cb]);
          pbu[cb][rb * 2 + (i >> 2)][i & 3] = w;
        }
      }
    };
    static_for<SCH::s.nm>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      static_for<TS::MAXL>([&](auto lc) {
        constexpr int f = SCH::s.fl[m][decltype(lc)::value];
        if constexpr (f >= 0) fr[f] = frag(f);
      });
      constexpr int f = SCH::s.mf[m];
      constexpr int ma = SCH::s.ma[m], mb = SCH::s.mb[m], mcb = SCH::s.mc[m];
      if constexpr (SCH::s.mt[m] == 0) {
        sacc[ma][mcb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[f], bq[mcb][mb], sacc[ma][mcb], 0, 0, 0);
      } else {
        oacc[mb][mcb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            fr[f], __builtin_bit_cast(bf16x8_t, pbu[mcb][ma]), oacc[mb][mcb], 0, 0, 0);
      }
      static_for<TS::MAXS>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        slice(ic<SCH::s.v[m][k]>{});
      });
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  auto tile_full = [&](auto Pc, int kt) __attribute__((always_inline)) { tile_sched(ic<kFull>{}, ic<1>{}, Pc, ic<0>{}, kt); };
  // Tile kt of parity P for a wave that sees part of it (generic path).
  // (With one V register set the transposition comes after the compute, so
  // the loads issued at the start of the tile have the tile to land.)
  auto tile_edge = [&](auto Pc, int kt) __attribute__((always_inline)) {
    constexpr int P = decltype(Pc)::value;
    kcopy(kt + 1, P ^ 1);
    __builtin_amdgcn_sched_barrier(0);  // the copies go out before the V loads
    gload(ic<lset(P)>{}, kt + VAHEAD);
    if (C::VS == 2 && kt + 1 <= kt1) stage(ic<sset(P)>{}, P ^ 1);
    compute_edge(P, kt);
    if (C::VS == 1 && kt + 1 <= kt1) stage(ic<sset(P)>{}, P ^ 1);
  };
  // Tile kt of parity P that this wave does not see: staging only.
  auto tile_empty = [&](auto Pc, int kt) __attribute__((always_inline)) {
    constexpr int P = decltype(Pc)::value;
    kcopy(kt + 1, P ^ 1);
    __builtin_amdgcn_sched_barrier(0);  // the copies go out before the V loads
    gload(ic<lset(P)>{}, kt + VAHEAD);
    if (kt + 1 <= kt1) stage(ic<sset(P)>{}, P ^ 1);
  };
  // End of a tile: this wave's LDS writes and k' copies have landed, then all
  // waves meet. Every tile body issues its NKD copies and then its 4*NVB V
  // loads (for a later tile), so "all but the 4*NVB newest loads"
  // is exactly the copies plus everything older; the V loads keep flying
  // across the barrier. The barrier is the bare instruction: the wait is
  // explicit, and the empty asm statements keep the compiler from moving
  // memory accesses across it.
  static_assert(4 * C::NVB <= 15, "the V loads of a tile fit the wait count");
  auto wg_barrier = [&]() __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  auto tile_sync = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0070 | (4 * C::NVB));  // vmcnt(4*NVB) lgkmcnt(0)
    wg_barrier();
  };
  // the same after a body that issued no copies or loads (the last tile)
  auto tile_sync_all = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    wg_barrier();
  };

  // ---- main loop: one barrier per tile; every wave runs kt0..kt1 and so
  // ---- meets every barrier. Each range of tiles of one kind runs its own
  // ---- loop, unrolled by two over the tile parity, so every loop body is
  // ---- straight-line.
  __syncthreads();  // every wave has read its q rows back
  stage(ic<0>{}, 0);
  tile_sync_all();
  auto run = [&](auto body, int ka, int kb_) __attribute__((always_inline)) {
    int kt = ka;
    if (kt <= kb_ && ((kt - kt0) & 1)) {
      body(ic<1>{}, kt);
      tile_sync();
      ++kt;
    }
    for (; kt + 1 <= kb_; kt += 2) {
      body(ic<0>{}, kt);
      tile_sync();
      body(ic<1>{}, kt + 1);
      tile_sync();
    }
    if (kt <= kb_) {
      body(ic<0>{}, kt);
      tile_sync();
    }
  };
  auto one = [&](auto body, int kt) __attribute__((always_inline)) {
    if ((kt - kt0) & 1) body(ic<1>{}, kt); else body(ic<0>{}, kt);
    tile_sync();
  };
  // Waves whose columns are 32*CB consecutive positions from a 32-key
  // boundary (a tile boundary when CB = 2; half H of a tile when CB = 1),
  // with a window that is a multiple of the tile or wider than the wave's
  // reach, see: nothing, then (if the window bites) one kWin tile, full
  // tiles, one kDiag tile (its own positions), then nothing.
  const bool aligned = hpw == 1 && (p.kofs & (32 * CB - 1)) == 0 && p.W >= C::BN &&
                       tw0 <= q_last && (p.W % C::BN == 0 || p.W >= tw0 + C::BN);
  // calls f(ic<H>) with the half of the tile where the wave's positions start
  auto with_half = [&](auto f) __attribute__((always_inline)) {
    if constexpr (C::CB == 1) {
      if ((tw0 / 32) & 1) f(ic<1>{}); else f(ic<0>{});
    } else {
      f(ic<0>{});
    }
  };
  // (A slice of the key tiles runs the part of this order inside [kt0, kt1].)
  if (!SPLIT && aligned) {
    const int ktD = tw0 / C::BN;
    const int ktW = tw0 - p.W >= 0 ? (tw0 - p.W) / C::BN : -1;
    const int kf0 = ktW >= 0 ? ktW + 1 : kt0;
    run(tile_empty, kt0, kf0 - 1 - (ktW >= 0 ? 1 : 0));
    if (ktW >= 0)
      with_half([&](auto Hc) {
        one([&](auto Pc, int kt) { tile_sched(ic<kWin>{}, ic<1>{}, Pc, Hc, kt); }, ktW);
      });
    run(tile_full, kf0, ktD - 1);
    with_half([&](auto Hc) {
      if (ktD < kt1) {
        one([&](auto Pc, int kt) { tile_sched(ic<kDiag>{}, ic<1>{}, Pc, Hc, kt); }, ktD);
      } else {
        if ((ktD - kt0) & 1) tile_sched(ic<kDiag>{}, ic<0>{}, ic<1>{}, Hc, ktD);
        else tile_sched(ic<kDiag>{}, ic<0>{}, ic<0>{}, Hc, ktD);
        tile_sync_all();
      }
    });
    run(tile_empty, ktD + 1, kt1);
  } else if (aligned) {
    const int ktD = tw0 / C::BN;
    const int ktW = tw0 - p.W >= 0 ? (tw0 - p.W) / C::BN : -1;
    const int kf0 = max(kt0, ktW + 1);
    run(tile_empty, kt0, min(kt1, ktW - 1));
    if (ktW >= kt0 && ktW <= kt1)
      with_half([&](auto Hc) {
        one([&](auto Pc, int kt) { tile_sched(ic<kWin>{}, ic<1>{}, Pc, Hc, kt); }, ktW);
      });
    run(tile_full, kf0, min(kt1, ktD - 1));
    if (ktD >= kt0 && ktD <= kt1)
      with_half([&](auto Hc) {
        if (ktD < kt1) {
          one([&](auto Pc, int kt) { tile_sched(ic<kDiag>{}, ic<1>{}, Pc, Hc, kt); }, ktD);
        } else {
          if ((ktD - kt0) & 1) tile_sched(ic<kDiag>{}, ic<0>{}, ic<1>{}, Hc, ktD);
          else tile_sched(ic<kDiag>{}, ic<0>{}, ic<0>{}, Hc, ktD);
          tile_sync_all();
        }
      });
    run(tile_empty, max(kt0, ktD + 1), kt1);
  } else {
    // full tiles for this wave: j0 + BN - 1 <= tw0 and tw1 - j0 < W
    const int ktA = max(kt0, tw1 - p.W + C::BN > 0 ? (tw1 - p.W + C::BN) / C::BN : 0);
    const int ktB = min(kt1, (tw0 + 1) / C::BN - 1);
    if (ktA <= ktB) {
      run(tile_edge, kt0, ktA - 1);
      run(tile_full, ktA, ktB);
      run(tile_edge, ktB + 1, kt1);
    } else {
      run(tile_edge, kt0, kt1);
    }
  }

  // ---- epilogue of a slice: its unnormalised fp32 output rows (lane-half hf
  // ---- holds dims 8*r4 + 4*hf .. +3 of each 32-dim block) and row sums
  if constexpr (SPLIT) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const float l = sum_halves(lsum[cb]);
      if (t[cb] < q_end) {
        const size_t row = (size_t)(qo_row0 + t[cb]) * p.H + h[cb];
        float* const orow = part_o() + row * D + 4 * hf;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4)
            st16(orow + db * 32 + 8 * r4,
                 u32x4_t{__float_as_uint(oacc[db][cb][4 * r4]), __float_as_uint(oacc[db][cb][4 * r4 + 1]),
                         __float_as_uint(oacc[db][cb][4 * r4 + 2]), __float_as_uint(oacc[db][cb][4 * r4 + 3])});
        if (hf == 0) part_l()[row] = l;
      }
    }
    return;
  }
  // ---- epilogue: normalise by the row sum, write the wave's output rows to
  // ---- its LDS rows (the last barrier of the tile loop freed the buffers),
  // ---- and store them row-major, CPR lanes per row, bf16 (B, T, H, D)
  {
    uint16_t* const os = qs;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      lsum[cb] = sum_halves(lsum[cb]);
      const float inv_l = 1.0f / lsum[cb];
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d = db * 32 + 8 * r4 + 4 * hf;
          const u32x2_t w = {pack_bf2(oacc[db][cb][4 * r4] * inv_l, oacc[db][cb][4 * r4 + 1] * inv_l),
                             pack_bf2(oacc[db][cb][4 * r4 + 2] * inv_l, oacc[db][cb][4 * r4 + 3] * inv_l)};
          st8(os + (cb * 32 + n) * C::QLD + d, w);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < C::NQL; ++i) {
      const int r = i * RPI + qr0;
      int tr, hr;
      col_row(r, tr, hr);
      const u32x4_t w = ld16(os + r * C::QLD + qc * 8);
      if (tr < q_end) st16_nt(og + ((size_t)(qo_row0 + tr) * p.H + hr) * D + qc * 8, w);
    }
    // the scores were exponentiated as 2^(s log2 e), so the row sum is the
    // natural-exponent softmax denominator and ln of it the row log-sum-exp
    if (LSE == kLseIfGiven && p.lse != nullptr && hf == 0) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
        if (t[cb] < q_end) p.lse[(size_t)(qo_row0 + t[cb]) * p.H + h[cb]] = __builtin_amdgcn_logf(lsum[cb]) * kLn2;
    }
  }
}

template <int D, int NW>
constexpr bool fwd_has_lse() { return !(D == 128 && NW >= 4); }
// resident bf16 workgroups per compute unit
template <int D, int NW>
constexpr int wg_per_cu() { return (NW == 2 || NW == 4) ? 2 : 1; }
template <int D, int NW>
__global__ void __launch_bounds__(64 * NW, (wg_per_cu<D, NW>())) attn_fwd_bf16_kernel(FwdArgs p) {
  attn_fwd_bf16_body<D, NW, false, fwd_has_lse<D, NW>() ? kLseIfGiven : kLseNone>(p);
}
template <int D, int NW>
__global__ void __launch_bounds__(64 * NW, (wg_per_cu<D, NW>())) attn_fwd_bf16_split_kernel(FwdArgs p) {
  attn_fwd_bf16_body<D, NW, true>(p);
}

// Sum of the slices of a split launch: o = (sum_s O_s) / (sum_s l_s), bf16.
// Scores are bounded by QK-norm, so the slices share one scale (no running
// maximum) and their partial sums add directly. One thread per 4 dims.
template <int D>
__global__ void __launch_bounds__(256) attn_split_combine_kernel(const float* __restrict__ part,
                                                                 uint16_t* __restrict__ o,
                                                                 float* __restrict__ lse,
                                                                 int rows, int nsplit) {
  constexpr int TPR = D / 4;  // threads per row
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = i / TPR;
  if (row >= rows) return;
  const int c4 = (int)(i - row * TPR);
  const float* pl = part + (size_t)nsplit * rows * D;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f, l = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const u32x4_t w = ld16(part + ((size_t)s * rows + row) * D + 4 * c4);
    a0 += __uint_as_float(w[0]);
    a1 += __uint_as_float(w[1]);
    a2 += __uint_as_float(w[2]);
    a3 += __uint_as_float(w[3]);
    l += pl[(size_t)s * rows + row];
  }
  const float inv = 1.0f / l;
  st8(o + row * D + 4 * c4, u32x2_t{pack_bf2(a0 * inv, a1 * inv), pack_bf2(a2 * inv, a3 * inv)});
  if (lse != nullptr && c4 == 0) lse[row] = __builtin_amdgcn_logf(l) * kLn2;
}

// =====================================================================
// fp32 kernel: one thread per query column, fp32 FMAs, k'/V tiles in LDS.
// =====================================================================
template <int D>
__global__ void __launch_bounds__(128) attn_fwd_f32_kernel(FwdArgs p) {
  constexpr int NT = 128, BN = 32;
  __shared__ float Kf[BN][D + 1];
  __shared__ float Vf[BN][D + 1];

  const float* __restrict__ qg = (const float*)p.q;
  const float* __restrict__ kg = (const float*)p.kp;
  const float* __restrict__ vg = (const float*)p.v;
  float* __restrict__ og = (float*)p.o;

  const int tid = threadIdx.x;
  const int per_qt = p.B * p.H;
  const int qt = p.nqt - 1 - (int)blockIdx.x / per_qt;
  const int rem = (int)blockIdx.x % per_qt;
  const int b = rem / p.H, h = rem - (rem / p.H) * p.H;
  const int g = h / p.G;
  const int q0 = qt * NT;
  const int q_last = min(q0 + NT, p.T) - 1 + p.kofs;  // a position (= key row)
  const int t = q0 + tid;
  const bool tvalid = t < p.T;
  const int tc = tvalid ? t : p.T - 1;
  const int ta = t + p.kofs;  // position of query row t

  float qv[D];
  {
    const float* qrow = qg + (((size_t)b * p.T + tc) * p.H + h) * D;
    const float2* trow = reinterpret_cast<const float2*>(p.tabq) + (size_t)tc * (D / 2);
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < D / 2; ++i) {
      const float2 cs = p.tabq != nullptr ? trow[i] : make_float2(1.f, 0.f);
      const float xe = qrow[2 * i], xo = qrow[2 * i + 1];
      const float ye = xe * cs.x - xo * cs.y, yo = xe * cs.y + xo * cs.x;
      qv[2 * i] = ye;
      qv[2 * i + 1] = yo;
      ss += ye * ye + yo * yo;
    }
    const float sc = p.tabq != nullptr ? p.qscale / sqrtf(ss * (1.0f / D) + kEps) : p.qscale;
#pragma unroll
    for (int d = 0; d < D; ++d) qv[d] *= sc;
  }

  float acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.f;
  float lsum = 0.f;

  const int k_first = max(0, q0 + p.kofs - p.W + 1);
  const int k_end = p.kofs + p.T;
  const size_t kv_row = (size_t)p.Hkv * D;
  for (int j0 = (k_first / BN) * BN; j0 <= q_last; j0 += BN) {
    __syncthreads();
    // stage K' and V: 4 threads per key row
    {
      const int r = tid >> 2, part = tid & 3;
      const int key = j0 + r;
      if (key < k_end) {
        const float* krow = kg + ((size_t)b * p.Tk + key) * kv_row + (size_t)g * D + part * (D / 4);
        const float* vrow = vg + ((size_t)b * p.Tk + key) * kv_row + (size_t)g * D + part * (D / 4);
#pragma unroll
        for (int i = 0; i < D / 4; ++i) {
          Kf[r][part * (D / 4) + i] = krow[i];
          Vf[r][part * (D / 4) + i] = vrow[i];
        }
      } else {
#pragma unroll
        for (int i = 0; i < D / 4; ++i) {
          Kf[r][part * (D / 4) + i] = 0.f;
          Vf[r][part * (D / 4) + i] = 0.f;
        }
      }
    }
    __syncthreads();
#pragma unroll 1
    for (int jj = 0; jj < BN; ++jj) {
      const int key = j0 + jj;
      const int dl = ta - key;
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
    if (p.lse != nullptr) p.lse[((size_t)b * p.T + t) * p.H + h] = logf(lsum);
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

// Waves per workgroup of the bf16 kernel. The full band: 8 waves, two per
// SIMD, one 32-column block each (256 columns, one workgroup per compute
// unit). Against one wave per SIMD with two blocks: 8-16% faster on the GQA
// D = 64 layers; at D = 128, with a fragment look-ahead of 3 MFMAs so that it
// fits 256 registers, 58.8-59.6 us against 62.4-62.7 us on the d12 L layer.
// A window of at most half the sequence gives every query tile about the
// same number of key tiles, and 1.5 tiles of 256 columns per compute unit
// leave half the units idle for the last round. There 4 waves of one block
// (128 columns) run as two workgroups per unit, again two waves per SIMD, and
// one workgroup's loads and stores overlap the other's tiles: d12 W = 512
// layer 49.1 -> 37.1 us (against the 2-wave form, one wave per SIMD with two
// blocks, which stays at D = 128 for log-sum-exp calls);
// GQA W = 512 layer 103 -> 97 us. On the full band the 256-column form is
// faster (GQA W = 2048: 167 us against 168-172).
template <int D>
constexpr int fwd_waves() { return 8; }
// (For a chunk whose queries start at position kofs, the window bites for
// most of its query tiles once it is at most kofs + T/2: 2W <= T + 2 kofs.
// Measured on a 512-token d12 chunk at offset 1536 with W = 512: 30.2 us with
// two waves against 32.1.)
static bool fwd_narrow(int T, int W, int kofs) {
  return 2 * (long long)W <= T + 2 * (long long)kofs;
}

// Key-tile slices. A launch of fewer workgroups than half the device holds
// leaves compute units idle while each workgroup walks its band of key tiles
// alone (a short prompt, a batch of one, a chunk at a large offset); there
// each query tile's key tiles are cut into nsplit slices, one workgroup each,
// so that up to a full device of workgroups run, every slice keeps at least
// kMinSliceTiles tiles, and a second kernel adds the slices up. The second
// kernel and each slice's own set-up cost a few microseconds, so bands
// shorter than 3 * kMinSliceTiles tiles are not cut (measured on d12-shaped
// launches: a batch of one at T = 2048 takes 37 us in 4 slices against 62
// whole; a 512-token chunk at offset 1536, 52 us in 2 slices against 62; a
// chunk at offset 512, 16 tiles, 40.6 us in 2 slices against 38.4 whole).
constexpr int kCUs = 256;  // compute units of the MI355X
constexpr int kMinSliceTiles = 8;
constexpr int kMaxSplits = 16;

static int fwd_splits(long long grid, int cap, int tiles) {
  if (grid <= 0 || 2 * grid > cap || tiles < 3 * kMinSliceTiles) return 1;
  int ns = (int)(cap / grid);
  ns = min(ns, tiles / kMinSliceTiles);
  ns = min(ns, kMaxSplits);
  return max(ns, 1);
}
// key tiles of the heaviest query tile (one of the last two)
static int max_key_tiles(const FwdArgs& a) {
  const int np = 1 << a.bp_log2;
  int best = 0;
  for (int qt = max(0, a.nqt - 2); qt < a.nqt; ++qt) {
    const int q0 = qt * np + a.kofs;
    const int ql = min(q0 + np, a.kofs + a.T) - 1;
    const int kf = max(0, q0 - a.W + 1);
    best = max(best, ql / 64 - kf / 64 + 1);
  }
  return best;
}
static size_t part_bytes_for(int nsplit, long long rows, int D) {
  return nsplit > 1 ? (size_t)nsplit * (size_t)rows * (size_t)(D + 1) * sizeof(float) : 0;
}

// Sliced D = 128 launches use the 4-wave kernel of 128 columns (two
// workgroups per compute unit), whose registers hold the slice bookkeeping
// (242 VGPRs; the 8-wave one is at 256 without it). Measured on the d12
// 512-token chunk at offset 1536, W = 2048: 48.5 us against 53.9 with the
// 2-wave form.
template <int D, int NW>
constexpr bool fwd_can_split() { return !(D == 128 && NW == 8); }

template <int D, int NW>
static long long bf16_grid(int B, int T, int H, int hpw) {
  using C = BfCfg<D, NW>;
  const int np = C::NC / hpw;
  return (long long)((T + np - 1) / np) * B * (H / hpw);
}

// query tiles of the NW-wave kernel in a, and the slices it would cut
template <int D, int NW>
static int plan_bf16(FwdArgs& a, int hpw, size_t part_bytes) {
  using C = BfCfg<D, NW>;
  a.bp_log2 = ilog2(C::NC / hpw);
  a.nqt = (a.T + (1 << a.bp_log2) - 1) >> a.bp_log2;
  if (!fwd_can_split<D, NW>() || a.part == nullptr) return 1;
  const int ns = fwd_splits((long long)a.nqt * a.B * a.ngroups, kCUs * wg_per_cu<D, NW>(), max_key_tiles(a));
  return part_bytes_for(ns, a.rows, D) > part_bytes ? 1 : ns;
}

template <int D, int NW>
static hipError_t launch_bf16(FwdArgs a, int hpw, size_t part_bytes, hipStream_t stream) {
  using C = BfCfg<D, NW>;
  a.nsplit = plan_bf16<D, NW>(a, hpw, part_bytes);
  const long long grid = (long long)a.nqt * a.B * a.ngroups;
  if (grid * a.nsplit > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (a.nsplit == 1) {
    if (!fwd_has_lse<D, NW>() && a.lse != nullptr) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, NW>), dim3((unsigned)grid), dim3(C::NT), 0, stream, a);
    return hipGetLastError();
  }
  if constexpr (fwd_can_split<D, NW>()) {
    hipLaunchKernelGGL((attn_fwd_bf16_split_kernel<D, NW>), dim3((unsigned)(grid * a.nsplit)),
                       dim3(C::NT), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long threads = (long long)a.rows * (D / 4);
    hipLaunchKernelGGL(attn_split_combine_kernel<D>, dim3((unsigned)((threads + 255) / 256)), dim3(256),
                       0, stream, (const float*)a.part, (uint16_t*)a.o, a.lse, a.rows, a.nsplit);
    return hipGetLastError();
  } else {
    return hipErrorInvalidConfiguration;
  }
}

// heads per workgroup of the bf16 kernel: largest power of two dividing G, at most 32
static int heads_per_wg(int G) {
  int hpw = 1;
  while (hpw < 32 && (G % (hpw * 2)) == 0) hpw *= 2;
  return hpw;
}

template <int D>
static size_t part_bytes_d(int B, int T, int H, int Hkv, int Tk) {
  const int hpw = heads_per_wg(H / Hkv);
  const int tiles = Tk / 64 + 2;  // at least the key tiles of any query tile
  int ns = 1;
  if constexpr (fwd_can_split<D, fwd_waves<D>()>())
    ns = fwd_splits(bf16_grid<D, fwd_waves<D>()>(B, T, H, hpw), kCUs * wg_per_cu<D, fwd_waves<D>()>(), tiles);
  constexpr int NWN = 4;  // the narrow-band and sliced form
  ns = max(ns, fwd_splits(bf16_grid<D, NWN>(B, T, H, hpw), kCUs * wg_per_cu<D, NWN>(), tiles));
  return part_bytes_for(ns, (long long)B * T * H, D);
}

template <int D>
static hipError_t attn_fwd_d(FwdArgs a, Dtype dt, size_t part_bytes, hipStream_t stream) {
  a.qscale = kLog2e / sqrtf((float)D);
  if (dt == kBF16) {
    const int hpw = heads_per_wg(a.G);
    a.hpw_log2 = ilog2(hpw);
    a.ngroups = a.H / hpw;
    if constexpr (D == 128) {
      // the row log-sum-exp: the 2-wave form; the narrow band or a launch cut
      // into slices: 4 waves of one column block, two workgroups per unit
      FwdArgs a2 = a;
      if (a.lse != nullptr) return launch_bf16<D, 2>(a, hpw, part_bytes, stream);
      if (fwd_narrow(a.T, a.W, a.kofs) || plan_bf16<D, 4>(a2, hpw, part_bytes) > 1)
        return launch_bf16<D, 4>(a, hpw, part_bytes, stream);
    } else {
      // the narrow band: 4 waves of one column block, two workgroups per unit
      if (fwd_narrow(a.T, a.W, a.kofs)) return launch_bf16<D, 4>(a, hpw, part_bytes, stream);
    }
    return launch_bf16<D, fwd_waves<D>()>(a, hpw, part_bytes, stream);
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

size_t attn_core_part_bytes(int B, int T, int H, int Hkv, int D, int Tk, Dtype dt) {
  if (dt != kBF16 || B < 1 || T < 1 || H < 1 || Hkv < 1 || H % Hkv != 0 || Tk < T) return 0;
  switch (D) {
    case 32: return part_bytes_d<32>(B, T, H, Hkv, Tk);
    case 64: return part_bytes_d<64>(B, T, H, Hkv, Tk);
    case 128: return part_bytes_d<128>(B, T, H, Hkv, Tk);
    default: return 0;
  }
}

hipError_t launch_attn_core(const void* q, const void* kp, const void* v, void* o, int B, int T,
                            int H, int Hkv, int D, int window, const void* tabq, int Tk, int kofs,
                            void* part, size_t part_bytes, Dtype dt, hipStream_t stream, float* lse) {
  FwdArgs a{};
  a.lse = lse;
  a.q = q;
  a.kp = kp;
  a.v = v;
  a.o = o;
  a.tabq = tabq;
  a.B = B;
  a.T = T;
  a.H = H;
  a.Hkv = Hkv;
  a.W = window;
  a.kofs = kofs;
  a.Tk = Tk;
  a.G = H / Hkv;
  a.rows = B * T * H;
  a.part = part_bytes > 0 ? (float*)part : nullptr;
  switch (D) {
    case 32: return attn_fwd_d<32>(a, dt, part_bytes, stream);
    case 64: return attn_fwd_d<64>(a, dt, part_bytes, stream);
    case 128: return attn_fwd_d<128>(a, dt, part_bytes, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace nc
