// Fused-Softmax attention forward on gfx950 scaled MFMA (MXFP8/6/4).
//
// What is computed (Fused-Softmax for efficient quantized attention, summary;
// Moving softmax to matrix operations speeds up AI inference by over 2x,
// "Read it as" and the "How it works" figure), with the readings fixed in the
// oracle's module documentation:
//   1. frozen max per query row from the first 128 keys: max(window max,
//      mean + (sqrt(2 ln n) + 1) * std) + bias;
//   2. S^T = K^ Q^T on the matrix cores with the accumulator initialised to
//      -m~: the max subtraction is folded into the product;
//   3. epilogue per 32-key MX block: block binade from the block's largest
//      score, then per element one FMA + one truncating conversion gives the
//      fp32 bit-pattern exponential 2^(t + shift), and the scaled conversion
//      rounds it onto the element grid: the exponential and the MX
//      quantisation of P in one pass, with no exp instruction;
//   4. O^T += V^T P~^T and l += 1 P~^T on the matrix cores (same P~ in
//      numerator and denominator, as EFQ-Softmax: Exp-Free Quantization for
//      Softmax, abstract, uses it);
//   5. a row whose block overflows the top binade is re-based by whole
//      binades: its running O and l are scaled by an exact power of two and
//      the remaining blocks use the raised reference (the fallback);
//   6. out = bf16(O / l).
//
// Work decomposition.  One workgroup = 4 waves = 4*16*NSUB query rows of one
// (batch, head).  Key tiles of 128 keys (K^ rows and the matching V^T
// columns) are staged in LDS and shared by the 4 waves.  Each wave keeps its
// queries' Q^ fragments, O^T accumulators and row sums in registers; there is
// no online max and no rescaling except on fallback.
//
// Register layout (16x16x128 scaled MFMA).  Lane (g, r) = 16g + r.  The score
// tile is computed transposed (keys as rows, queries as columns) so that a
// lane ends up with 32 keys of one query: the K^ rows are gathered from LDS
// in the order that makes those 32 keys exactly the keys this lane must
// supply as the B operand of the P V product.  For FP6/FP4 that is one whole
// MX block of P; for FP8 it is two half blocks, completed with the lane
// 16 apart.
#include "fsa_device.h"
#include "fsa_internal.h"

namespace fsa {

namespace {

constexpr int KT = 128;          // keys per tile
constexpr int NWAVES = 4;
constexpr float MAGIC = 12582912.0f;   // 1.5 * 2^23: float + MAGIC rounds to an integer

__device__ __forceinline__ uint32_t cvt_u32_trunc(float y) {
  // Truncation toward zero with saturation; negative and NaN give 0.
  uint32_t u;
  asm volatile("v_cvt_u32_f32 %0, %1" : "=v"(u) : "v"(y));
  return u;
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFF + ((u >> 16) & 1);
  return (uint16_t)(u >> 16);
}

// Position p (0..31) of a lane's operand list -> key (or K index) within the
// 128-wide K dimension, for lane group g.
template <int F>
__device__ __forceinline__ int kpos(int g, int p) {
  if (Fmt<F>::bits == 8) return p < 16 ? 16 * g + p : 64 + 16 * g + (p - 16);
  return 32 * g + p;
}

// Copy a lane's operand bytes for one row from LDS: the 32 K elements this
// lane group holds along a row of D (or 128) elements.  `row` points at the
// row's first byte; `len` is the row's valid element count (elements past it
// read as zero codes).
template <int F>
__device__ __forceinline__ v8i load_operand(const uint8_t* row, int g, int len) {
  v8i o = {0, 0, 0, 0, 0, 0, 0, 0};
  if (Fmt<F>::bits == 8) {
    if (16 * g < len) {
      uint4 a = *reinterpret_cast<const uint4*>(row + 16 * g);
      o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    }
    if (64 + 16 * g < len) {
      uint4 b = *reinterpret_cast<const uint4*>(row + 64 + 16 * g);
      o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
    }
  } else if (Fmt<F>::bits == 6) {
    if (32 * g < len) {
      const uint2* p = reinterpret_cast<const uint2*>(row + 24 * g);
      uint2 a = p[0], b = p[1], c = p[2];
      o[0] = a.x; o[1] = a.y; o[2] = b.x; o[3] = b.y; o[4] = c.x; o[5] = c.y;
    }
  } else {
    if (32 * g < len) {
      uint4 a = *reinterpret_cast<const uint4*>(row + 16 * g);
      o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    }
  }
  return o;
}

template <int F>
__device__ __forceinline__ v4f mfma(const v8i& a, const v8i& b, const v4f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, Fmt<F>::mfma, Fmt<F>::mfma,
                                                          0, sa, 0, sb);
}

template <int F>
__device__ __forceinline__ v8i ones_operand() {
  constexpr int BITS = Fmt<F>::bits;
  constexpr uint32_t c = Fmt<F>::one_code;
  v8i o = {0, 0, 0, 0, 0, 0, 0, 0};
  if (BITS == 8) {
    for (int i = 0; i < 8; ++i) o[i] = (int)(c * 0x01010101u);
  } else if (BITS == 4) {
    for (int i = 0; i < 4; ++i) o[i] = (int)(c * 0x11111111u);
  } else {
    // 32 six-bit fields: 4 fields make 3 bytes, repeated.
    const uint32_t w24 = c | (c << 6) | (c << 12) | (c << 18);
    const uint8_t b0 = w24 & 0xFF, b1 = (w24 >> 8) & 0xFF, b2 = (w24 >> 16) & 0xFF;
    uint8_t bytes[24];
    for (int i = 0; i < 8; ++i) { bytes[3 * i] = b0; bytes[3 * i + 1] = b1; bytes[3 * i + 2] = b2; }
    for (int i = 0; i < 6; ++i)
      o[i] = (int)(bytes[4 * i] | (bytes[4 * i + 1] << 8) | (bytes[4 * i + 2] << 16) |
                   ((uint32_t)bytes[4 * i + 3] << 24));
  }
  return o;
}

}  // namespace

template <int F, int D, bool CAUSAL, int NSUB>
__global__ void __launch_bounds__(256, 1) fsa_fwd_kernel(AttnArgs a) {
  constexpr int BITS = Fmt<F>::bits;
  constexpr int MB = Fmt<F>::mbits;
  constexpr int EMAX = Fmt<F>::emax;
  constexpr int ETOP = Fmt<F>::e_top;
  constexpr int CAP = 127 - EMAX;
  constexpr int RB = D * BITS / 8;          // bytes per Q^/K^ row
  constexpr int VRB = KT * BITS / 8;        // bytes per V^T tile row
  constexpr int NDB = D / 32;               // MX blocks per Q^/K^ row
  constexpr int NDT = D / 16;               // 16-wide output tiles along D
  constexpr int KRS = RB + 16;              // LDS row stride (padded)
  constexpr int VRS = VRB + 16;
  constexpr int QW = NWAVES * 16 * NSUB;    // queries per workgroup

  __shared__ __align__(16) uint8_t k_lds[KT * KRS];
  __shared__ __align__(16) uint8_t ks_lds[KT * NDB];
  __shared__ __align__(16) uint8_t v_lds[D * VRS];
  __shared__ __align__(16) uint32_t vs_lds[D];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int r = lane & 15;

  // workspace slabs are indexed by the launch's own (batch, head) order;
  // outputs by the global head index
  const int64_t wi = blockIdx.y;
  const int b = blockIdx.y / a.hrun;
  const int h = a.h0 + (blockIdx.y - b * a.hrun);
  const int64_t bh = (int64_t)b * a.H + h;
  const int S = a.S;
  const int q_wg = blockIdx.x * QW;
  const int q_wave = q_wg + wave * 16 * NSUB;

  const uint8_t* kc = a.kc + wi * (int64_t)a.sk_alloc * RB;
  const uint8_t* ks = a.ks + wi * (int64_t)a.sk_alloc * NDB;
  const int64_t v_row = (int64_t)a.sk_alloc * BITS / 8;
  const uint8_t* vc = a.vc + wi * (int64_t)D * v_row;
  const int vs_row = a.sk_alloc / 32;
  const uint8_t* vs = a.vs + wi * (int64_t)D * vs_row;

  // ---- Q^ fragments (B operand of the score product), one per subtile
  v8i qf[NSUB];
  int qsc[NSUB];
  {
    const uint8_t* qc = a.qc + wi * (int64_t)a.sq_alloc * RB;
    const uint8_t* qs = a.qs + wi * (int64_t)a.sq_alloc * NDB;
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      const int q = q_wave + 16 * s + r;
      qf[s] = load_operand<F>(qc + (int64_t)q * RB, g, D);
      qsc[s] = g < NDB ? (int)qs[(int64_t)q * NDB + g] : 127;
    }
  }

  // ---- key-tile range
  int n_tiles = (S + KT - 1) / KT;
  if (CAUSAL) {
    const int last_q = q_wg + QW - 1 < S - 1 ? q_wg + QW - 1 : S - 1;
    const int t_need = last_q / KT + 1;
    n_tiles = t_need < n_tiles ? t_need : n_tiles;
  }

  auto load_tile = [&](int t) {
    // K^ rows [t*KT, t*KT+KT): contiguous in global memory
    constexpr int KCH = KT * RB / 16;
    const uint8_t* src = kc + (int64_t)t * KT * RB;
    for (int c = tid; c < KCH; c += 256) {
      const int row = c / (RB / 16), col = c - row * (RB / 16);
      *reinterpret_cast<uint4*>(k_lds + row * KRS + col * 16) =
          *reinterpret_cast<const uint4*>(src + (int64_t)c * 16);
    }
    constexpr int KSCH = KT * NDB / 16;
    const uint8_t* ssrc = ks + (int64_t)t * KT * NDB;
    for (int c = tid; c < KSCH; c += 256)
      *reinterpret_cast<uint4*>(ks_lds + c * 16) = *reinterpret_cast<const uint4*>(ssrc + c * 16);
    // V^T rows d in [0, D), columns = this tile's keys
    constexpr int VCH = D * VRB / 16;
    for (int c = tid; c < VCH; c += 256) {
      const int row = c / (VRB / 16), col = c - row * (VRB / 16);
      *reinterpret_cast<uint4*>(v_lds + row * VRS + col * 16) =
          *reinterpret_cast<const uint4*>(vc + row * v_row + (int64_t)t * VRB + col * 16);
    }
    if (tid < D)
      vs_lds[tid] = *reinterpret_cast<const uint32_t*>(vs + (int64_t)tid * vs_row + t * (KT / 32));
  };

  // A operand of the score product for 16-key slice j: row R of the slice is
  // key kpos(R/4, 4j + R%4) of the tile, so that output row 4g+i lands on the
  // lane's operand position 4j+i.
  auto k_frag = [&](int j, int& sc) -> v8i {
    const int kk = kpos<F>(r >> 2, 4 * j + (r & 3));
    sc = g < NDB ? (int)ks_lds[kk * NDB + g] : 127;
    return load_operand<F>(k_lds + kk * KRS, g, D);
  };

  const v4f zero4 = {0.f, 0.f, 0.f, 0.f};

  // ---- frozen max from the first tile (keys [0, 128))
  float mg[NSUB];
  {
    __syncthreads();
    load_tile(0);
    __syncthreads();
    v4f acc[NSUB][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int sc;
      const v8i kf = k_frag(j, sc);
#pragma unroll
      for (int s = 0; s < NSUB; ++s) acc[s][j] = mfma<F>(kf, qf[s], zero4, sc, qsc[s]);
    }
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      const int q = q_wave + 16 * s + r;
      float sum = 0.f, mx = -INFINITY;
      int cnt = 0;
#pragma unroll
      for (int p = 0; p < 32; ++p) {
        const int key = kpos<F>(g, p);
        const bool vis = key < S && (!CAUSAL || key <= q);
        const float x = acc[s][p >> 2][p & 3];
        sum += vis ? x : 0.f;
        mx = vis ? __builtin_fmaxf(mx, x) : mx;
        cnt += vis ? 1 : 0;
      }
      sum += __shfl_xor(sum, 16); sum += __shfl_xor(sum, 32);
      cnt += __shfl_xor(cnt, 16); cnt += __shfl_xor(cnt, 32);
      mx = __builtin_fmaxf(mx, __shfl_xor(mx, 16)); mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
      const float mean = sum / (float)(cnt > 0 ? cnt : 1);
      float ss = 0.f;
#pragma unroll
      for (int p = 0; p < 32; ++p) {
        const int key = kpos<F>(g, p);
        const bool vis = key < S && (!CAUSAL || key <= q);
        const float dlt = acc[s][p >> 2][p & 3] - mean;
        ss += vis ? dlt * dlt : 0.f;
      }
      ss += __shfl_xor(ss, 16); ss += __shfl_xor(ss, 32);
      const float sd = __builtin_sqrtf(ss / (float)(cnt > 0 ? cnt : 1));
      const int nvis = CAUSAL ? (q + 1 < S ? q + 1 : S) : S;
      const float z = __builtin_sqrtf(2.0f * __builtin_logf((float)nvis)) + 1.0f;
      mg[s] = __builtin_fmaxf(mx, mean + z * sd) + a.bias;
    }
  }

  // ---- main sweep
  v4f O[NSUB][NDT];
  v4f L[NSUB];
  int kap[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    L[s] = zero4;
    kap[s] = 0;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) O[s][dt] = zero4;
  }
  const v8i ones = ones_operand<F>();
  const float alpha = a.alpha, beta = a.beta;
  const float gmin = -2097152.0f / alpha;    // keeps alpha*g inside the MAGIC window

  for (int t = 0; t < n_tiles; ++t) {
    if (t > 0) {
      __syncthreads();
      load_tile(t);
      __syncthreads();
    }
    const int key0 = t * KT;
    const bool need_mask = (key0 + KT > S) || (CAUSAL && key0 + KT - 1 > q_wave);

    v4f acc[NSUB][8];
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      const v4f init = {-mg[s], -mg[s], -mg[s], -mg[s]};
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[s][j] = init;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int sc;
      const v8i kf = k_frag(j, sc);
#pragma unroll
      for (int s = 0; s < NSUB; ++s) acc[s][j] = mfma<F>(kf, qf[s], acc[s][j], sc, qsc[s]);
    }

    v8i pw[NSUB];
    int psc[NSUB];
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      float x[32];
#pragma unroll
      for (int p = 0; p < 32; ++p) x[p] = acc[s][p >> 2][p & 3];
      if (need_mask) {
        const int q = q_wave + 16 * s + r;
#pragma unroll
        for (int p = 0; p < 32; ++p) {
          const int key = key0 + kpos<F>(g, p);
          const bool vis = key < S && (!CAUSAL || key <= q);
          x[p] = vis ? x[p] : -INFINITY;
        }
      }
      // block maxima: one block per lane (FP6/FP4) or two half blocks (FP8)
      float m0 = x[0], m1 = x[16];
#pragma unroll
      for (int p = 1; p < 16; ++p) { m0 = __builtin_fmaxf(m0, x[p]); m1 = __builtin_fmaxf(m1, x[16 + p]); }
      if (BITS == 8) {
        m0 = __builtin_fmaxf(m0, __shfl_xor(m0, 16));
        m1 = __builtin_fmaxf(m1, __shfl_xor(m1, 16));
      } else {
        m0 = __builtin_fmaxf(m0, m1);
        m1 = m0;
      }
      // block binade E = e_top + floor(round(alpha * max) / 2^M)
      auto binade = [&](float m) -> int {
        const float mc = __builtin_fmaxf(m, gmin);
        const float tt = __builtin_fmaf(alpha, mc, MAGIC);
        const int c = (int)(__float_as_uint(tt) - __float_as_uint(MAGIC));
        return ETOP + (c >> MB);
      };
      int E0 = binade(m0), E1 = binade(m1);
      // fallback: any block above the top binade re-bases its row
      const bool over = (E0 - kap[s] > ETOP) || (E1 - kap[s] > ETOP);
      if (__builtin_amdgcn_ballot_w64(over) != 0) {
        int em = E0 > E1 ? E0 : E1;
        em = max(em, __shfl_xor(em, 16));
        em = max(em, __shfl_xor(em, 32));
        const int nk = max(kap[s], em - ETOP);
        if (nk != kap[s]) {
          const float f = __builtin_ldexpf(1.0f, kap[s] - nk);
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) O[s][dt] *= f;
          L[s] *= f;
          kap[s] = nk;
        }
      }
      const int d0 = min(ETOP - (E0 - kap[s]), CAP);
      const int d1 = min(ETOP - (E1 - kap[s]), CAP);
      const float base0 = (float)(127 + EMAX + d0 - kap[s]) * 8388608.0f;
      const float base1 = (float)(127 + EMAX + d1 - kap[s]) * 8388608.0f;
      float pv[32];
#pragma unroll
      for (int p = 0; p < 32; ++p) {
        const float y = __builtin_fmaf(beta, x[p], p < 16 ? base0 : base1);
        pv[p] = __uint_as_float(cvt_u32_trunc(y));
      }
      uint32_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      Pack32<F>::run(pv, w);
#pragma unroll
      for (int i = 0; i < 8; ++i) pw[s][i] = (int)w[i];
      const int s0 = 127 - EMAX - d0, s1 = 127 - EMAX - d1;
      if (BITS == 8) {
        // lane group c supplies the scale of key block c: blocks 0/2 live in
        // groups 0-1 (low/high half), blocks 1/3 in groups 2-3.
        const int o0 = __shfl_xor(s0, 48), o1 = __shfl_xor(s1, 48);
        psc[s] = g == 0 ? s0 : (g == 1 ? o0 : (g == 2 ? o1 : s1));
      } else {
        psc[s] = s0;
      }
    }

    // P V and the row sums on the matrix cores
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int d = 16 * dt + r;
      const v8i vf = load_operand<F>(v_lds + d * VRS, g, KT);
      const int vsc = (int)((vs_lds[d] >> (8 * g)) & 0xFF);
#pragma unroll
      for (int s = 0; s < NSUB; ++s) O[s][dt] = mfma<F>(vf, pw[s], O[s][dt], vsc, psc[s]);
    }
#pragma unroll
    for (int s = 0; s < NSUB; ++s) L[s] = mfma<F>(ones, pw[s], L[s], 127, psc[s]);
  }

  // ---- normalise and store: lane (g, r) holds O[q][16dt + 4g + i]
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    const int q = q_wave + 16 * s + r;
    if (q < S) {
      const float inv = 1.0f / L[s][0];
      uint16_t* orow = a.out + (bh * S + q) * (int64_t)D;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const uint32_t lo = f32_to_bf16_rne(O[s][dt][0] * inv) | ((uint32_t)f32_to_bf16_rne(O[s][dt][1] * inv) << 16);
        const uint32_t hi = f32_to_bf16_rne(O[s][dt][2] * inv) | ((uint32_t)f32_to_bf16_rne(O[s][dt][3] * inv) << 16);
        *reinterpret_cast<uint2*>(orow + 16 * dt + 4 * g) = make_uint2(lo, hi);
      }
      if (g == 0) {
        if (a.row_kappa) a.row_kappa[bh * S + q] = kap[s];
        if (a.row_mguess) a.row_mguess[bh * S + q] = mg[s];
      }
    }
  }
}

template <int F, int D, bool CAUSAL>
static hipError_t launch3(const AttnArgs& a, hipStream_t stream) {
  constexpr int NSUB = 2;
  constexpr int QW = NWAVES * 16 * NSUB;
  dim3 grid((a.S + QW - 1) / QW, a.B * a.hrun);
  hipLaunchKernelGGL((fsa_fwd_kernel<F, D, CAUSAL, NSUB>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int F>
static hipError_t launch2(const AttnArgs& a, int D, int causal, hipStream_t stream) {
  if (D == 128) return causal ? launch3<F, 128, true>(a, stream) : launch3<F, 128, false>(a, stream);
  return causal ? launch3<F, 64, true>(a, stream) : launch3<F, 64, false>(a, stream);
}

int fsa_queries_per_workgroup() { return NWAVES * 16 * 2; }

hipError_t launch_fsa_fwd(const AttnArgs& a, int fmt, int D, int causal, hipStream_t stream) {
  if (fmt == FMT_E4M3) return launch2<FMT_E4M3>(a, D, causal, stream);
  if (fmt == FMT_E2M3) return launch2<FMT_E2M3>(a, D, causal, stream);
  return launch2<FMT_E2M1>(a, D, causal, stream);
}

}  // namespace fsa
