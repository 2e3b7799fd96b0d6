// Fused bias-free q, k, v projection with the RoPE and QK-norm epilogue, for
// gfx950: the GEMM directly before the attention forward.
//
// What is computed ("从文本到聊天模型" (onehacker.top) §5.4: q = c_q(x),
// k = c_k(x), v = c_v(x) viewed as (B, T, H, D) and (B, T, Hkv, D);
// "Nanochat与nanoGPT对比：关键升级" (lzwjava.github.io) §1 table: linear layers
// without bias, QK-norm after RoPE; §5.6 of the first page: RoPE):
//   q' = RMSNorm(RoPE(x w_q^T)),  k' = RMSNorm(RoPE(x w_k^T)),  v = x w_v^T,
// weights in the linear-layer layout (out_features, in_features), output
// column h*D + d being element d of head h, positions pos_offset + t.
//
// Design (bf16 path): the product is formed transposed, C^T = W x^T, with
// v_mfma_f32_32x32x16_bf16, the weight rows as the A operand and the token
// rows as the B operand. In the accumulator a lane then holds one token and
// half of a head's D dims (32 db + 8 (r/4) + 4 hf + r%4), so the epilogue
// works on fp32 accumulators in registers: the RoPE pairs (d, d+1) sit in the
// same lane, and the RMSNorm sum needs one cross-lane add (lanes n, n + 32).
// Nothing round-trips through memory between the product and q', k'.
//  * A workgroup owns 256 tokens (4 waves x 64) and a group of 128 weight
//    rows: one head at D = 128, two at 64, four at 32 (a group stays inside
//    one of the three matrices; rows of heads past its last read as zero and
//    are not stored). Every weight fragment read from LDS feeds two MFMAs
//    (two 32-token blocks).
//  * The x and weight tiles of each 32-column chunk of the input dimension go
//    memory -> LDS with 16-byte buffer-to-LDS copies (no registers),
//    double-buffered, one barrier per chunk; rows of 64 bytes are XOR-
//    swizzled so the row-strided fragment reads spread over all LDS banks.
//    48 KB of LDS and 168 registers per wave, so three workgroups share a
//    compute unit and hide each other's waits.
//  * XCD-aware order: workgroup b runs on XCD b mod 8; XCD x takes a
//    contiguous run of token blocks, and within it all row groups of a token
//    block back to back, so the block's x rows are read from HBM once into
//    that XCD's L2 and served from there to every group.
// fp32 path: exact fp32 arithmetic on the vector ALUs, one thread per
// (token, head), not a performance path.
#include "device_common.hpp"
#include "launch.hpp"

namespace nc {

struct QkvArgs {
  const void* x;                   // (M, C), M = B*T tokens
  const void* wq, *wk, *wv;        // (H*D, C), (Hkv*D, C), (Hkv*D, C)
  void* q, *k, *v;                 // (M, H, D), (M, Hkv, D), (M, Hkv, D)
  const void* tab;                 // (cos, sin) of positions pos_offset + t: [T][D/2]
  int M, T, C, H, Hkv, NH;         // NH = H + 2 Hkv output heads
  int ntb, tbx;                    // token blocks; token blocks per XCD
  int ngq, ngk, NG;                // row groups of w_q, of w_k (= of w_v); NG = ngq + 2 ngk
};

template <int D>
struct QkvCfg {
  static constexpr int NW = 4, CB = 2;
  static constexpr int BT = 64 * NW;            // tokens per workgroup
  static constexpr int RG = 128;                // weight rows (output columns) per workgroup
  static constexpr int HPG = RG / D;            // heads per row group
  static constexpr int KC = 32;                 // input columns per LDS chunk
  static constexpr int CPRK = KC / 8;           // 16-byte chunks per tile row
  static constexpr int RPS = 256 / (KC * 2);    // tile rows per 256-byte span of the LDS banks
  static constexpr int DB = RG / 32;            // 32-row blocks of the group
  static constexpr int DBH = D / 32;            // of one head
  static constexpr int XT = BT * KC;            // bf16 elements of the x tile
  static constexpr int WT = RG * KC;            // of the weight tile
  static constexpr int STAGE = XT + WT;
  static constexpr int XCOPY = XT * 2 / 1024;   // 1 KB copies per x tile
  static constexpr int WCOPY = WT * 2 / 1024;   // per weight tile
  static constexpr int CPWMAX = (XCOPY + WCOPY + NW - 1) / NW;  // copies per wave per chunk, at most
};

// LDS chunk of logical 16-byte chunk c of row r in a tile of KC-column rows:
// chunk c of row r sits at c ^ ((r / RPS) mod CPRK), so the rows of a 16-row
// fragment read land on distinct 16-byte bank groups
template <int D>
__device__ __forceinline__ int q_chunk(int r, int c) {
  using C = QkvCfg<D>;
  return r * C::CPRK + (c ^ ((r / C::RPS) % C::CPRK));
}

// row group -> (matrix, its head count, first head of the group)
struct HeadSel {
  const uint16_t* w;
  uint16_t* out;
  int nh, hh;
  bool rot;
};

template <int D>
__global__ void __launch_bounds__(256, 2) qkv_bf16_kernel(QkvArgs p) {
  using C = QkvCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * C::STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hf = lane >> 5;

  const int bx = (int)blockIdx.x;
  const int xcd = bx & 7, l = bx >> 3;
  const int tb = xcd * p.tbx + l / p.NG;
  const int grp = l % p.NG;
  if (tb >= p.ntb || l / p.NG >= p.tbx) return;  // padding of the XCD ranges

  HeadSel hs;
  if (grp < p.ngq) {
    hs = {(const uint16_t*)p.wq, (uint16_t*)p.q, p.H, grp * C::HPG, true};
  } else if (grp < p.ngq + p.ngk) {
    hs = {(const uint16_t*)p.wk, (uint16_t*)p.k, p.Hkv, (grp - p.ngq) * C::HPG, true};
  } else {
    hs = {(const uint16_t*)p.wv, (uint16_t*)p.v, p.Hkv, (grp - p.ngq - p.ngk) * C::HPG, false};
  }
  const int m0 = tb * C::BT;
  const uint32_t rowb = (uint32_t)p.C * 2;
  const __amdgpu_buffer_rsrc_t rx =
      make_rsrc((const uint16_t*)p.x + (size_t)m0 * p.C, (uint32_t)min(C::BT, p.M - m0) * rowb);
  // rows of heads past the matrix's last read as zero, and are not stored
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(hs.w + (size_t)hs.hh * D * p.C,
                                              (uint32_t)(min(C::HPG, hs.nh - hs.hh) * D) * rowb);
  const int nkc = p.C / C::KC;

  // Copy f (x tile first, then the weight tile) is issued by wave f mod NW:
  // this wave's copies are f = i*NW + wave, and only their offsets are kept.
  auto issue = [&](int kc, int buf) __attribute__((always_inline)) {
    uint16_t* st = smem + buf * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::CPWMAX; ++i) {
      const int f = i * C::NW + wave;
      if (f >= C::XCOPY + C::WCOPY) break;  // uniform
      const bool isx = f < C::XCOPY;
      const int ff = isx ? f : f - C::XCOPY;
      const int e = ff * 64 + lane;
      const int r = e / C::CPRK, c = e % C::CPRK;
      const uint32_t off = (uint32_t)r * rowb + (uint32_t)kc * (C::KC * 2) +
                           (uint32_t)((c ^ ((r / C::RPS) % C::CPRK)) * 16);
      if (isx) lds_copy16(rx, st + ff * 512, off);
      else lds_copy16(rw, st + C::XT + ff * 512, off);
    }
  };
  auto sync = [&]() __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  f32x16_t acc[C::DB][C::CB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][cb][r] = 0.f;

  issue(0, 0);
  sync();
  for (int kc = 0; kc < nkc; ++kc) {
    const int buf = kc & 1;
    if (kc + 1 < nkc) issue(kc + 1, buf ^ 1);
    const uint16_t* xs = smem + buf * C::STAGE;
    const uint16_t* ws = xs + C::XT;
#pragma unroll
    for (int s = 0; s < C::KC / 16; ++s) {
      bf16x8_t xb[C::CB];
#pragma unroll
      for (int cb = 0; cb < C::CB; ++cb)
        xb[cb] = *reinterpret_cast<const bf16x8_t*>(xs + q_chunk<D>(wave * 64 + cb * 32 + n, 2 * s + hf) * 8);
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const bf16x8_t wa = *reinterpret_cast<const bf16x8_t*>(ws + q_chunk<D>(db * 32 + n, 2 * s + hf) * 8);
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb)
          acc[db][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa, xb[cb], acc[db][cb], 0, 0, 0);
      }
    }
    sync();
  }

  // ---- epilogue: the lane holds token m, group rows 32 db + 8 (r/4) + 4 hf + r%4;
  // head j of the group is row blocks db = j*DBH .. j*DBH + DBH-1
  const uint32_t* tab = (const uint32_t*)p.tab;
#pragma unroll
  for (int cb = 0; cb < C::CB; ++cb) {
    const int m = m0 + wave * 64 + cb * 32 + n;
    const bool valid = m < p.M;
    const int t = (valid ? m : 0) % p.T;
#pragma unroll
    for (int j = 0; j < C::HPG; ++j) {
      if (hs.hh + j >= hs.nh) break;  // uniform
      uint16_t* orow = hs.out + ((size_t)(valid ? m : 0) * hs.nh + hs.hh + j) * D;
      float y[C::DBH][16];
      if (hs.rot) {
        float ss = 0.f;
#pragma unroll
        for (int dh = 0; dh < C::DBH; ++dh)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int d = dh * 32 + 8 * r4 + 4 * hf;
            const u32x2_t cs = *reinterpret_cast<const u32x2_t*>(tab + (size_t)t * (D / 2) + d / 2);
#pragma unroll
            for (int mm = 0; mm < 2; ++mm) {
              const float xe = acc[j * C::DBH + dh][cb][4 * r4 + 2 * mm];
              const float xo = acc[j * C::DBH + dh][cb][4 * r4 + 2 * mm + 1];
              const float c = h_lo(cs[mm]), sn = h_hi(cs[mm]);
              const float ye = xe * c - xo * sn, yo = xe * sn + xo * c;
              y[dh][4 * r4 + 2 * mm] = ye;
              y[dh][4 * r4 + 2 * mm + 1] = yo;
              ss += ye * ye + yo * yo;
            }
          }
        const float rn = rsq(sum_halves(ss) * (1.0f / D) + kEps);
#pragma unroll
        for (int dh = 0; dh < C::DBH; ++dh)
#pragma unroll
          for (int r = 0; r < 16; ++r) y[dh][r] *= rn;
      } else {
#pragma unroll
        for (int dh = 0; dh < C::DBH; ++dh)
#pragma unroll
          for (int r = 0; r < 16; ++r) y[dh][r] = acc[j * C::DBH + dh][cb][r];
      }
#pragma unroll
      for (int dh = 0; dh < C::DBH; ++dh)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const u32x2_t w = {pack_bf2(y[dh][4 * r4], y[dh][4 * r4 + 1]),
                             pack_bf2(y[dh][4 * r4 + 2], y[dh][4 * r4 + 3])};
          if (valid) st8(orow + dh * 32 + 8 * r4 + 4 * hf, w);
        }
    }
  }
}

// fp32: one thread per (token, output head), exact fp32 arithmetic
template <int D>
__global__ void __launch_bounds__(64) qkv_f32_kernel(QkvArgs p) {
  const long long idx = (long long)blockIdx.x * 64 + threadIdx.x;
  if (idx >= (long long)p.M * p.NH) return;
  const int m = (int)(idx / p.NH), head = (int)(idx % p.NH);
  const float* w;
  float* out;
  int nh, hh;
  bool rot = true;
  if (head < p.H) {
    w = (const float*)p.wq; out = (float*)p.q; nh = p.H; hh = head;
  } else if (head < p.H + p.Hkv) {
    w = (const float*)p.wk; out = (float*)p.k; nh = p.Hkv; hh = head - p.H;
  } else {
    w = (const float*)p.wv; out = (float*)p.v; nh = p.Hkv; hh = head - p.H - p.Hkv; rot = false;
  }
  const float* xr = (const float*)p.x + (size_t)m * p.C;
  const float* wr = w + (size_t)hh * D * p.C;
  float acc[D];
  for (int d = 0; d < D; ++d) acc[d] = 0.f;
  for (int c = 0; c < p.C; ++c) {
    const float xv = xr[c];
    for (int d = 0; d < D; ++d) acc[d] += xv * wr[(size_t)d * p.C + c];
  }
  float* orow = out + ((size_t)m * nh + hh) * D;
  if (rot) {
    const float2* tr = (const float2*)p.tab + (size_t)(m % p.T) * (D / 2);
    float ss = 0.f;
    for (int i = 0; i < D / 2; ++i) {
      const float2 cs = tr[i];
      const float xe = acc[2 * i], xo = acc[2 * i + 1];
      acc[2 * i] = xe * cs.x - xo * cs.y;
      acc[2 * i + 1] = xe * cs.y + xo * cs.x;
      ss += acc[2 * i] * acc[2 * i] + acc[2 * i + 1] * acc[2 * i + 1];
    }
    const float rn = 1.0f / sqrtf(ss * (1.0f / D) + kEps);
    for (int d = 0; d < D; ++d) orow[d] = acc[d] * rn;
  } else {
    for (int d = 0; d < D; ++d) orow[d] = acc[d];
  }
}

template <int D>
static hipError_t qkv_d(QkvArgs a, Dtype dt, hipStream_t stream) {
  if (dt == kBF16) {
    using C = QkvCfg<D>;
    a.ntb = (a.M + C::BT - 1) / C::BT;
    a.tbx = (a.ntb + 7) / 8;
    a.ngq = (a.H + C::HPG - 1) / C::HPG;
    a.ngk = (a.Hkv + C::HPG - 1) / C::HPG;
    a.NG = a.ngq + 2 * a.ngk;
    const long long grid = 8LL * a.tbx * a.NG;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(qkv_bf16_kernel<D>, dim3((unsigned)grid), dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  const long long n = (long long)a.M * a.NH;
  if ((n + 63) / 64 > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(qkv_f32_kernel<D>, dim3((unsigned)((n + 63) / 64)), dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_qkv_rope_qknorm(const void* x, const void* wq, const void* wk, const void* wv,
                                  void* q, void* k, void* v, const void* tab, int B, int T, int C,
                                  int H, int Hkv, int D, Dtype dt, hipStream_t stream) {
  QkvArgs a{};
  a.x = x;
  a.wq = wq;
  a.wk = wk;
  a.wv = wv;
  a.q = q;
  a.k = k;
  a.v = v;
  a.tab = tab;
  a.M = B * T;
  a.T = T;
  a.C = C;
  a.H = H;
  a.Hkv = Hkv;
  a.NH = H + 2 * Hkv;
  switch (D) {
    case 32: return qkv_d<32>(a, dt, stream);
    case 64: return qkv_d<64>(a, dt, stream);
    case 128: return qkv_d<128>(a, dt, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace nc
