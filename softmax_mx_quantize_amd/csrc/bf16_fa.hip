// Plain BF16 flash attention on gfx950: the in-house baseline.
//
// This is the "BF16 attention" the fused-softmax kernels are compared with
// (Fused-Softmax for efficient quantized attention, summary) and the
// "Softmax (Vector)" path of the "How it works" figure in Moving softmax to
// matrix operations speeds up AI inference by over 2x: bf16 products on the
// matrix cores with fp32 accumulation, and a softmax on the vector units with
// an exact exponential, an online row max and rescaling of the running
// output whenever the max grows.
//
// Work decomposition mirrors the fused kernel: a workgroup of 4 waves covers
// 4*16*NSUB query rows of one (batch, head); 64-key tiles of K (row-major)
// and V (transposed while staging) live in LDS.  Scores are computed
// transposed (keys x queries) with 16x16x32 bf16 MFMAs so that each lane
// owns the keys of one query; P is fed back as the B operand of
// O^T = V^T P^T without leaving registers.  The pairing of K positions
// between the two operands of each product is chosen here (the hardware's
// internal K order is irrelevant because both operands use the same one).
#include "fsa_device.h"
#include "fsa_internal.h"

namespace fsa {

namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int BKT = 64;          // keys per tile
constexpr int BWAVES = 4;

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
  ua += 0x7FFF + ((ua >> 16) & 1);
  ub += 0x7FFF + ((ub >> 16) & 1);
  return (ua >> 16) | (ub & 0xFFFF0000u);
}

__device__ __forceinline__ v4f mfma_bf16(const v4i& a, const v4i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a),
                                                 __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}

}  // namespace

template <int D, bool CAUSAL, int NSUB>
__global__ void __launch_bounds__(256, 1) bf16_fa_kernel(Bf16Args a) {
  constexpr int KRS = D * 2 + 16;        // bytes per K row in LDS (padded)
  constexpr int VRS = BKT * 2 + 16;      // bytes per V^T row in LDS (padded)
  constexpr int NDS = D / 32;            // 32-wide steps along D
  constexpr int NDT = D / 16;
  constexpr int QW = BWAVES * 16 * NSUB;

  __shared__ __align__(16) uint8_t k_lds[BKT * KRS];
  __shared__ __align__(16) uint8_t v_lds[D * VRS];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, g = lane >> 4, r = lane & 15;
  const int64_t bh = blockIdx.y;
  const int S = a.S;
  const int q_wg = blockIdx.x * QW;
  const int q_wave = q_wg + wave * 16 * NSUB;
  const uint16_t* qg = a.q + bh * (int64_t)S * D;
  const uint16_t* kg = a.k + bh * (int64_t)S * D;
  const uint16_t* vg = a.v + bh * (int64_t)S * D;

  // Q fragments: column = query, K positions = d in [32ds + 8g, +8)
  v4i qf[NSUB][NDS];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    const int q = q_wave + 16 * s + r;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      v4i z = {0, 0, 0, 0};
      if (q < S) {
        uint4 u = *reinterpret_cast<const uint4*>(qg + (int64_t)q * D + 32 * ds + 8 * g);
        z[0] = u.x; z[1] = u.y; z[2] = u.z; z[3] = u.w;
      }
      qf[s][ds] = z;
    }
  }

  int n_tiles = (S + BKT - 1) / BKT;
  if (CAUSAL) {
    const int last_q = q_wg + QW - 1 < S - 1 ? q_wg + QW - 1 : S - 1;
    const int t_need = last_q / BKT + 1;
    n_tiles = t_need < n_tiles ? t_need : n_tiles;
  }

  const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
  v4f O[NSUB][NDT];
  float m_run[NSUB], l_run[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    m_run[s] = -INFINITY;
    l_run[s] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) O[s][dt] = zero4;
  }
  const float sl2 = a.scale_log2;

  for (int t = 0; t < n_tiles; ++t) {
    const int key0 = t * BKT;
    __syncthreads();
    // K tile: rows key0.., row-major; zero rows past S
    {
      constexpr int CH = BKT * D * 2 / 16;
      for (int c = tid; c < CH; c += 256) {
        const int row = c / (D / 8), col = c - row * (D / 8);
        uint4 u = make_uint4(0, 0, 0, 0);
        if (key0 + row < S) u = *reinterpret_cast<const uint4*>(kg + (int64_t)(key0 + row) * D + col * 8);
        *reinterpret_cast<uint4*>(k_lds + row * KRS + col * 16) = u;
      }
    }
    // V tile transposed: thread takes keys (2k, 2k+1) x 8 d, writes 8 key pairs
    {
      constexpr int CH = (BKT / 2) * (D / 8);
      for (int c = tid; c < CH; c += 256) {
        const int kp = c / (D / 8), col = c - kp * (D / 8);
        const int k0 = key0 + 2 * kp;
        uint4 u0 = make_uint4(0, 0, 0, 0), u1 = make_uint4(0, 0, 0, 0);
        if (k0 < S) u0 = *reinterpret_cast<const uint4*>(vg + (int64_t)k0 * D + col * 8);
        if (k0 + 1 < S) u1 = *reinterpret_cast<const uint4*>(vg + (int64_t)(k0 + 1) * D + col * 8);
        const uint32_t a0[4] = {u0.x, u0.y, u0.z, u0.w};
        const uint32_t a1[4] = {u1.x, u1.y, u1.z, u1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t lo = (a0[e >> 1] >> (16 * (e & 1))) & 0xFFFF;
          const uint32_t hi = (a1[e >> 1] >> (16 * (e & 1))) & 0xFFFF;
          *reinterpret_cast<uint32_t*>(v_lds + (col * 8 + e) * VRS + 4 * kp) = lo | (hi << 16);
        }
      }
    }
    __syncthreads();
    const bool need_mask = (key0 + BKT > S) || (CAUSAL && key0 + BKT - 1 > q_wave);

    // S^T slices j = 0..3 (16 keys each)
    v4f sc[NSUB][4];
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
      for (int j = 0; j < 4; ++j) sc[s][j] = zero4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        const uint4 u = *reinterpret_cast<const uint4*>(k_lds + (16 * j + r) * KRS + (32 * ds + 8 * g) * 2);
        const v4i kf = {(int)u.x, (int)u.y, (int)u.z, (int)u.w};
#pragma unroll
        for (int s = 0; s < NSUB; ++s) sc[s][j] = mfma_bf16(kf, qf[s][ds], sc[s][j]);
      }
    }

    v4i pf[NSUB][2];
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      const int q = q_wave + 16 * s + r;
      float x[16];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = sc[s][j][i] * sl2;
          if (need_mask) {
            const int key = key0 + 16 * j + 4 * g + i;
            const bool vis = key < S && (!CAUSAL || key <= q);
            v = vis ? v : -INFINITY;
          }
          x[4 * j + i] = v;
        }
      float tm = x[0];
#pragma unroll
      for (int p = 1; p < 16; ++p) tm = __builtin_fmaxf(tm, x[p]);
      tm = __builtin_fmaxf(tm, __shfl_xor(tm, 16));
      tm = __builtin_fmaxf(tm, __shfl_xor(tm, 32));
      const float m_new = __builtin_fmaxf(m_run[s], tm);
      const float corr = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run[s] - m_new);
      m_run[s] = m_new;
      const float msub = m_new == -INFINITY ? 0.0f : m_new;
      float ps = 0.f;
#pragma unroll
      for (int p = 0; p < 16; ++p) {
        x[p] = __builtin_amdgcn_exp2f(x[p] - msub);
        ps += x[p];
      }
      l_run[s] = l_run[s] * corr + ps;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) O[s][dt] *= corr;
      // B operand positions: chunk c holds keys 32c + 4g + i (slice 2c) then
      // 32c + 16 + 4g + i (slice 2c+1)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        v4i z;
        z[0] = (int)pack_bf16x2(x[8 * c + 0], x[8 * c + 1]);
        z[1] = (int)pack_bf16x2(x[8 * c + 2], x[8 * c + 3]);
        z[2] = (int)pack_bf16x2(x[8 * c + 4], x[8 * c + 5]);
        z[3] = (int)pack_bf16x2(x[8 * c + 6], x[8 * c + 7]);
        pf[s][c] = z;
      }
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int d = 16 * dt + r;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const uint2 u0 = *reinterpret_cast<const uint2*>(v_lds + d * VRS + (32 * c + 4 * g) * 2);
        const uint2 u1 = *reinterpret_cast<const uint2*>(v_lds + d * VRS + (32 * c + 16 + 4 * g) * 2);
        const v4i vf = {(int)u0.x, (int)u0.y, (int)u1.x, (int)u1.y};
#pragma unroll
        for (int s = 0; s < NSUB; ++s) O[s][dt] = mfma_bf16(vf, pf[s][c], O[s][dt]);
      }
    }
  }

#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    float l = l_run[s];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int q = q_wave + 16 * s + r;
    if (q < S) {
      const float inv = 1.0f / l;
      uint16_t* orow = a.out + (bh * S + q) * (int64_t)D;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const uint32_t lo = pack_bf16x2(O[s][dt][0] * inv, O[s][dt][1] * inv);
        const uint32_t hi = pack_bf16x2(O[s][dt][2] * inv, O[s][dt][3] * inv);
        *reinterpret_cast<uint2*>(orow + 16 * dt + 4 * g) = make_uint2(lo, hi);
      }
    }
  }
}

template <int D, bool CAUSAL>
static hipError_t launch_b(const Bf16Args& a, hipStream_t stream) {
  constexpr int NSUB = 2;
  constexpr int QW = BWAVES * 16 * NSUB;
  dim3 grid((a.S + QW - 1) / QW, a.BH);
  hipLaunchKernelGGL((bf16_fa_kernel<D, CAUSAL, NSUB>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bf16_fa(const Bf16Args& a, int D, int causal, hipStream_t stream) {
  if (D == 128) return causal ? launch_b<128, true>(a, stream) : launch_b<128, false>(a, stream);
  return causal ? launch_b<64, true>(a, stream) : launch_b<64, false>(a, stream);
}

}  // namespace fsa
