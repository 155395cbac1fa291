// Plain BF16 flash attention on gfx950: the in-house baseline.
//
// This is the unquantised attention the fused-softmax kernels are compared
// with (Fused-Softmax for efficient quantized attention, summary) and the
// vector-unit softmax path of the "How it works" figure in Moving softmax to
// matrix operations speeds up AI inference by over 2x: bf16 products on the
// matrix cores with fp32 accumulation, and a softmax on the vector units with
// an exact exponential and a running row max that rescales the running output
// when it grows.
//
// It is built like the fused kernel so that the comparison measures the
// softmax and not the staging: a workgroup of 4 waves covers 128 query rows
// of one (batch, head), two workgroups share a CU, 64-key tiles of K and of
// V^T stream through two-stage LDS rings by direct buffer -> LDS loads, and
// the workgroups of one XCD sweep the same head.  V is transposed by a
// pre-pass into the workspace ([BH][D][S rounded up to 64], keys past S
// zero), so that both operands of the output product read 16-byte runs.
//
// Scores are computed transposed (keys x queries) with 16x16x32 bf16 MFMAs,
// so that a lane owns 4 keys of one query per 16-key slice.  The key order
// of the K rows is permuted (slice j, row m <-> tile key
// 32(j/2) + 8(m/4) + 4(j%2) + m%4) so that a lane's probabilities of slices
// 2c and 2c+1 are the 8 consecutive keys 32c + 8g .. +7: exactly the run
// its V^T operand of the output product O^T = V^T P^T reads.  The row sum
// comes from the same product with a ones operand.
//
// The running max is kept lazily: a tile raises it (and rescales O and the
// row sum) only when its max exceeds the kept one by more than 8 binades,
// so probabilities stay at most 2^8 and the rescale is rare.  The result
// is the same softmax; only the reference point of the exponentials moves.
#include "fsa_device.h"
#include "fsa_internal.h"
#include "lds_dma.h"

namespace fsa {

namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));

constexpr int BKT = BF16_KEY_TILE;          // keys per tile
constexpr int BWAVES = 4;
constexpr int BNSUB = 2;                    // 16-query subtiles per wave
constexpr int BQW = BWAVES * 16 * BNSUB;    // queries per workgroup
constexpr float LAZY_BINADES = 8.0f;

__device__ __forceinline__ v4f mfma_bf16(const v4i& a, const v4i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a),
                                                 __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}

// Two fp32 -> bf16 (round to nearest even) in one word, a in the low half.
__device__ __forceinline__ int pack_bf16x2(float a, float b) {
  const v2f f = {a, b};
  return __builtin_bit_cast(int, __builtin_convertvector(f, v2bf));
}

// Max over the four lane groups holding one query (lanes r, r+16, r+32,
// r+48), on the vector unit: the 32-lane swap pairs groups 0/2 and 1/3,
// the 16-lane swap then pairs the results.
__device__ __forceinline__ float group_max(float x) {
  const uint32_t xb = __float_as_uint(x);
  const auto h = __builtin_amdgcn_permlane32_swap(xb, xb, false, false);
  const float y = __builtin_fmaxf(__uint_as_float(h[0]), __uint_as_float(h[1]));
  const uint32_t yb = __float_as_uint(y);
  const auto q = __builtin_amdgcn_permlane16_swap(yb, yb, false, false);
  return __builtin_fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

// XOR swizzles of the 16-byte chunks of an LDS row, chosen so that the 16
// lanes of a lane group, which read the same logical chunk of 16 different
// rows, hit 16 distinct bank quads.  K rows are 2D bytes; a lane group
// reads rows whose bits 0-1 and 3-4 run through all values.
template <int D>
__device__ __forceinline__ int swz_krow(int rho) {
  if (D == 128) return (rho & 3) | (((rho >> 3) & 3) << 2);
  return ((rho >> 1) & 1) | (((rho >> 3) & 3) << 1);   // 128-byte rows, two per bank line
}
// V^T rows are 128 bytes (64 keys), two per bank line; a lane group reads
// 16 consecutive rows.
__device__ __forceinline__ int swz_vrow(int d) { return (d >> 1) & 7; }

// V [BH][S][D] -> V^T [BH][D][s_alloc]; keys S..s_alloc-1 are written zero.
template <int D>
__global__ void __launch_bounds__(256) bf16_vt_kernel(const uint16_t* __restrict__ v,
                                                      uint16_t* __restrict__ vt, int S, int s_alloc) {
  __shared__ uint16_t tl[64][64 + 2];   // [d][key]
  const int key0 = blockIdx.x * 64, d0 = blockIdx.y * 64;
  const int64_t bh = blockIdx.z;
  const uint16_t* src = v + bh * (int64_t)S * D;
  uint16_t* dst = vt + bh * (int64_t)D * s_alloc;
  for (int c = threadIdx.x; c < 512; c += 256) {
    const int key = c >> 3, dc = c & 7;
    uint4 u = make_uint4(0, 0, 0, 0);
    if (key0 + key < S)
      u = *reinterpret_cast<const uint4*>(src + (int64_t)(key0 + key) * D + d0 + 8 * dc);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) tl[8 * dc + e][key] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
  }
  __syncthreads();
  for (int c = threadIdx.x; c < 512; c += 256) {
    const int d = c >> 3, kc = c & 7;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (uint32_t)tl[d][8 * kc + 2 * e] | ((uint32_t)tl[d][8 * kc + 2 * e + 1] << 16);
    *reinterpret_cast<uint4*>(dst + (int64_t)(d0 + d) * s_alloc + key0 + 8 * kc) =
        make_uint4(w[0], w[1], w[2], w[3]);
  }
}

}  // namespace

template <int D, bool CAUSAL>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2)))
bf16_fa_kernel(Bf16Args a) {
#if defined(__HIP_DEVICE_COMPILE__)  // buffer-resource types exist only in the device pass
  constexpr int RB = 2 * D;                  // bytes per K row
  constexpr int K_TILE = BKT * RB;
  constexpr int VRB = 2 * BKT;               // bytes per V^T row of a tile
  constexpr int V_TILE = D * VRB;
  constexpr int NDS = D / 32;                // 32-wide steps along D (score product)
  constexpr int NDT = D / 16;                // 16-row tiles of O^T
  constexpr int NK_DMA = K_TILE / 1024 / BWAVES;   // 1 KB loads per wave and tile
  constexpr int NV_DMA = V_TILE / 1024 / BWAVES;
  static_assert(NK_DMA >= 1 && NV_DMA >= 1, "tile smaller than one load per wave");

  // Two-stage rings; each stage is its own LDS object addressed through a
  // compile-time index, so reads of one stage are not taken to alias the
  // loads in flight into the other.
  __shared__ __align__(16) uint8_t kl0[K_TILE];
  __shared__ __align__(16) uint8_t kl1[K_TILE];
  __shared__ __align__(16) uint8_t vl0[V_TILE];
  __shared__ __align__(16) uint8_t vl1[V_TILE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int r = lane & 15;

  // Workgroups are dealt round-robin to the 8 XCDs; each XCD takes a
  // contiguous run of (head, query tile) items so that its L2 serves one
  // head's K and V^T to all of them.
  const int S = a.S;
  const int nq = (S + BQW - 1) / BQW;
  const int n_items = nq * a.BH;
  const int per_xcd = (n_items + 7) / 8;
  const int item = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (item >= n_items) return;
  const int bh_i = item / nq;
  const int64_t bh = bh_i;
  const int q_wg = (item - bh_i * nq) * BQW;
  const int q_wave = q_wg + wave * 16 * BNSUB;

  const uint16_t* qg = a.q + bh * (int64_t)S * D;
  const uint16_t* kg = a.k + bh * (int64_t)S * D;
  const uint16_t* vtg = a.vt + bh * (int64_t)D * a.s_alloc;
  // K rows past S lie outside the resource and load as zeros.
  const __amdgpu_buffer_rsrc_t k_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)kg, (short)0, S * RB, 0x00020000);
  const __amdgpu_buffer_rsrc_t v_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)vtg, (short)0, D * a.s_alloc * 2, 0x00020000);

  // Load k of a wave fills LDS bytes [1024 (wave + 4k), +1024) of a stage:
  // lane i the physical chunk at 16 i, loaded from the logical chunk the
  // swizzle maps there.  The tile's offset is added to the lane offset (not
  // put in the scalar offset) so that the range check covers it.
  int k_voff[NK_DMA], v_voff[NV_DMA];
#pragma unroll
  for (int k = 0; k < NK_DMA; ++k) {
    const int b = (wave + BWAVES * k) * 1024 + 16 * lane;
    const int rho = b / RB, pc = (b % RB) / 16;
    k_voff[k] = rho * RB + (pc ^ swz_krow<D>(rho)) * 16;
  }
#pragma unroll
  for (int k = 0; k < NV_DMA; ++k) {
    const int b = (wave + BWAVES * k) * 1024 + 16 * lane;
    const int d = b / VRB, pc = (b % VRB) / 16;
    v_voff[k] = d * (a.s_alloc * 2) + (pc ^ swz_vrow(d)) * 16;
  }
  auto issue = [&](int t, uint8_t* kb, uint8_t* vb) __attribute__((always_inline)) {
    const uint32_t kla = lds_addr(kb), vla = lds_addr(vb);
#pragma unroll
    for (int k = 0; k < NK_DMA; ++k)
      dma_lds16(k_rsrc, kla + (wave + BWAVES * k) * 1024, k_voff[k] + t * K_TILE, 0);
#pragma unroll
    for (int k = 0; k < NV_DMA; ++k)
      dma_lds16(v_rsrc, vla + (wave + BWAVES * k) * 1024, v_voff[k] + t * VRB, 0);
  };

  int n_tiles = (S + BKT - 1) / BKT;
  if (CAUSAL) {
    const int last_q = q_wg + BQW - 1 < S - 1 ? q_wg + BQW - 1 : S - 1;
    const int t_need = last_q / BKT + 1;
    n_tiles = t_need < n_tiles ? t_need : n_tiles;
  }
  issue(0, kl0, vl0);

  // Q fragments (B operand of the score product): query r of the subtile,
  // d in [32 ds + 8 g, +8).
  v4i qf[BNSUB][NDS];
#pragma unroll
  for (int s = 0; s < BNSUB; ++s) {
    const int q = q_wave + 16 * s + r;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      v4i z = {0, 0, 0, 0};
      if (q < S) z = *reinterpret_cast<const v4i*>(qg + (int64_t)q * D + 32 * ds + 8 * g);
      qf[s][ds] = z;
    }
  }
  // Consume the fragments here: the compiler does not see the assembly
  // wait below, and would otherwise wait for them (vmcnt(0), so also for the
  // ring's prefetch) at their first use inside the sweep, on every tile.
#pragma unroll
  for (int s = 0; s < BNSUB; ++s)
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) asm volatile("" ::"v"(qf[s][ds]));

  const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
  const v4i ones = {0x3F803F80, 0x3F803F80, 0x3F803F80, 0x3F803F80};   // bf16 1.0 pairs
  v4f O[BNSUB][NDT];
  v4f L[BNSUB];
  float m_run[BNSUB], m_neg[BNSUB];
#pragma unroll
  for (int s = 0; s < BNSUB; ++s) {
    m_run[s] = -INFINITY;
    m_neg[s] = 0.f;
    L[s] = zero4;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) O[s][dt] = zero4;
  }
  const float sl2 = a.scale_log2;
  const float lazy_raw = LAZY_BINADES / sl2;   // the same margin in score units

  wait_dma();
  ring_barrier();
  if (n_tiles > 1) issue(1, kl1, vl1);

  auto step = [&](int t, auto st_tag) __attribute__((always_inline)) {
    constexpr int ST = decltype(st_tag)::value;
    uint8_t* kb = ST == 0 ? kl0 : kl1;
    uint8_t* vb = ST == 0 ? vl0 : vl1;
    const int key0 = t * BKT;
    // a causal wave whose queries all precede the tile has nothing to add
    const bool live = !CAUSAL || key0 <= q_wave + 16 * BNSUB - 1;
    if (live) {
      v4f sc[BNSUB][4];
#pragma unroll
      for (int s = 0; s < BNSUB; ++s)
#pragma unroll
        for (int j = 0; j < 4; ++j) sc[s][j] = zero4;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rho = 32 * (j >> 1) + 8 * (r >> 2) + 4 * (j & 1) + (r & 3);
        const uint8_t* krow = kb + rho * RB;
        const int sw = swz_krow<D>(rho);
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
          const v4i kf = *reinterpret_cast<const v4i*>(krow + ((4 * ds + g) ^ sw) * 16);
#pragma unroll
          for (int s = 0; s < BNSUB; ++s) sc[s][j] = mfma_bf16(kf, qf[s][ds], sc[s][j]);
        }
      }

      const bool need_mask = key0 + BKT > S || (CAUSAL && key0 + BKT - 1 > q_wave);
      v4i pf[BNSUB][2];
#pragma unroll
      for (int s = 0; s < BNSUB; ++s) {
        float x[4][4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) x[j][i] = sc[s][j][i];
        if (need_mask) {
          const int q = q_wave + 16 * s + r;
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int key = key0 + 32 * (j >> 1) + 8 * g + 4 * (j & 1) + i;
              const bool vis = key < S && (!CAUSAL || key <= q);
              x[j][i] = vis ? x[j][i] : -INFINITY;
            }
        }
        float tm = x[0][0];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) tm = __builtin_fmaxf(tm, x[j][i]);
        tm = group_max(tm);
        const bool grow = tm > m_run[s] + lazy_raw;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
          const float m_new = __builtin_fmaxf(m_run[s], tm);
          const float corr =
              m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f((m_run[s] - m_new) * sl2);
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) O[s][dt] *= corr;
          L[s] *= corr;
          m_run[s] = m_new;
          m_neg[s] = m_new == -INFINITY ? 0.0f : -m_new * sl2;
        }
        float p[4][4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            p[j][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[j][i], sl2, m_neg[s]));
        // B operand chunk c: keys 32c + 8g + 0..3 (slice 2c), then + 4..7
        // (slice 2c+1)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          v4i z;
          z[0] = pack_bf16x2(p[2 * c][0], p[2 * c][1]);
          z[1] = pack_bf16x2(p[2 * c][2], p[2 * c][3]);
          z[2] = pack_bf16x2(p[2 * c + 1][0], p[2 * c + 1][1]);
          z[3] = pack_bf16x2(p[2 * c + 1][2], p[2 * c + 1][3]);
          pf[s][c] = z;
        }
      }

#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int d = 16 * dt + r;
        const uint8_t* vrow = vb + d * VRB;
        const int sw = swz_vrow(d);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const v4i vf = *reinterpret_cast<const v4i*>(vrow + ((4 * c + g) ^ sw) * 16);
#pragma unroll
          for (int s = 0; s < BNSUB; ++s) O[s][dt] = mfma_bf16(vf, pf[s][c], O[s][dt]);
        }
      }
#pragma unroll
      for (int s = 0; s < BNSUB; ++s)
#pragma unroll
        for (int c = 0; c < 2; ++c) L[s] = mfma_bf16(ones, pf[s][c], L[s]);
    }
    // the next tile has landed (this wave's part) and every wave is done
    // with this stage: refill it two tiles ahead
    wait_dma();
    ring_barrier();
    if (t + 2 < n_tiles) issue(t + 2, kb, vb);
  };

  for (int t = 0; t < n_tiles; t += 2) {
    step(t, std::integral_constant<int, 0>{});
    if (t + 1 < n_tiles) step(t + 1, std::integral_constant<int, 1>{});
  }

  // every row of the row-sum product holds the full sum of its query
#pragma unroll
  for (int s = 0; s < BNSUB; ++s) {
    const int q = q_wave + 16 * s + r;
    if (q < S) {
      const float inv = 1.0f / L[s][0];
      uint16_t* orow = a.out + (bh * S + q) * (int64_t)D;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int lo = pack_bf16x2(O[s][dt][0] * inv, O[s][dt][1] * inv);
        const int hi = pack_bf16x2(O[s][dt][2] * inv, O[s][dt][3] * inv);
        *reinterpret_cast<uint2*>(orow + 16 * dt + 4 * g) = make_uint2((uint32_t)lo, (uint32_t)hi);
      }
    }
  }
#endif
}

template <int D, bool CAUSAL>
static hipError_t launch_b(const Bf16Args& a, hipStream_t stream) {
  hipLaunchKernelGGL((bf16_vt_kernel<D>), dim3(a.s_alloc / 64, D / 64, a.BH), dim3(256), 0, stream,
                     a.v, a.vt, a.S, a.s_alloc);
  const int n_items = (a.S + BQW - 1) / BQW * a.BH;
  hipLaunchKernelGGL((bf16_fa_kernel<D, CAUSAL>), dim3((n_items + 7) / 8 * 8), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bf16_fa(const Bf16Args& a, int D, int causal, hipStream_t stream) {
  if (D == 128) return causal ? launch_b<128, true>(a, stream) : launch_b<128, false>(a, stream);
  return causal ? launch_b<64, true>(a, stream) : launch_b<64, false>(a, stream);
}

}  // namespace fsa
