// C ABI of the fused-softmax MX attention library: argument validation,
// per-device workspace, launch sequencing and error mapping.  Declarations
// and the contract of every entry point are in include/fsa.h.
#include "fsa.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <mutex>
#include <new>
#include <unordered_map>
#include <vector>

#include "fsa_internal.h"

namespace {

constexpr int kKeyTile = 128;

int fmt_bits(int fmt) { return fmt == FSA_MXFP8_E4M3 ? 8 : (fmt == FSA_MXFP6_E2M3 ? 6 : 4); }
bool fmt_ok(int fmt) { return fmt == FSA_MXFP8_E4M3 || fmt == FSA_MXFP6_E2M3 || fmt == FSA_MXFP4_E2M1; }

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// fsa_fmt -> kernel format index
int kern_fmt(int fmt) { return fmt == FSA_MXFP8_E4M3 ? 0 : (fmt == FSA_MXFP6_E2M3 ? 1 : 2); }

struct Workspace {
  void* ptr = nullptr;
  size_t bytes = 0;
};

std::mutex g_mu;
std::unordered_map<int, Workspace> g_ws;

// Returns a device buffer of at least `need` bytes for the current device.
// Growing it synchronises the device first so that no enqueued kernel still
// reads the old buffer.
int workspace(size_t need, uint8_t** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FSA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  Workspace& w = g_ws[dev];
  if (w.bytes < need) {
    if (w.ptr) {
      if (hipDeviceSynchronize() != hipSuccess) return FSA_ERR_HIP;
      if (hipFree(w.ptr) != hipSuccess) return FSA_ERR_HIP;
      w.ptr = nullptr;
      w.bytes = 0;
    }
    const size_t sz = round_up((int64_t)need, 1 << 21);
    if (hipMalloc(&w.ptr, sz) != hipSuccess) {
      (void)hipGetLastError();
      w.ptr = nullptr;
      return FSA_ERR_NO_MEMORY;
    }
    w.bytes = sz;
  }
  *out = static_cast<uint8_t*>(w.ptr);
  return FSA_OK;
}

// Ids that tell the fallback pass whether its own call's first pass asked
// for it (the flag word keeps the last id that did).
uint64_t next_call_id() {
  static std::atomic<uint64_t> counter{0};
  return ++counter;
}

// Sub-allocation inside the workspace, 256-byte aligned.
struct Carver {
  size_t off = 0;
  size_t take(size_t n) {
    const size_t at = off;
    off = (size_t)round_up((int64_t)(off + n), 256);
    return at;
  }
};

struct RunLayout {
  int h0, hrun, fmt;
  size_t kc, ks, vc, vs;
};

int validate_attn(const void* q, const void* k, const void* v, void* out, int B, int H, int S,
                  int D, int causal) {
  if (!q || !k || !v || !out) return FSA_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || S <= 0 || D <= 0) return FSA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FSA_ERR_INVALID_ARG;
  const double total = (double)B * H * S * D;
  if (total > 1099511627776.0) return FSA_ERR_INVALID_ARG;  // 2^40 elements
  if ((int64_t)B * H > 65535) return FSA_ERR_INVALID_ARG;    // grid.y limit
  if (S > (1 << 30)) return FSA_ERR_INVALID_ARG;
  if (out == q || out == k || out == v) return FSA_ERR_INVALID_ARG;
  for (const void* p : {q, k, v, static_cast<const void*>(out)})
    if (reinterpret_cast<uintptr_t>(p) & 15) return FSA_ERR_INVALID_ARG;   // 16-byte vector loads
  if (D != 64 && D != 128) return FSA_ERR_UNSUPPORTED;
  // one head's bf16 rows (and its quantised slabs) are addressed with
  // 32-bit buffer offsets
  if (round_up(S, 128) * D * 2 >= ((int64_t)1 << 31)) return FSA_ERR_UNSUPPORTED;
  return FSA_OK;
}

int quantize(const uint16_t* x, uint8_t* codes, uint8_t* scales, int64_t batch, int64_t rows,
             int64_t cols, int64_t out_rows, int64_t nb_out, int64_t code_stride,
             int64_t scale_stride, int fmt, int mode, hipStream_t stream, float mult = 1.0f,
             int scale_layout = fsa::SCALES_ROWS) {
  fsa::QuantArgs a;
  a.x = x;
  a.codes = codes;
  a.scales = scales;
  a.batch = batch;
  a.rows = rows;
  a.cols = cols;
  a.out_rows = out_rows;
  a.nb_out = nb_out;
  a.code_stride = code_stride;
  a.scale_stride = scale_stride;
  a.batch0 = 0;
  a.mult = mult;
  a.scale_layout = scale_layout;
  return fsa::launch_mx_quant(a, fmt, mode, stream) == hipSuccess ? FSA_OK : FSA_ERR_HIP;
}

}  // namespace

extern "C" {

const char* fsa_strerror(int status) {
  switch (status) {
    case FSA_OK: return "success";
    case FSA_ERR_INVALID_ARG: return "invalid argument";
    case FSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case FSA_ERR_HIP: return "HIP runtime or launch error";
    case FSA_ERR_NO_MEMORY: return "device memory allocation failed";
    default: return "unknown status";
  }
}

int fsa_quantize_mx(const void* x_bf16, void* codes, void* scales_e8m0, int64_t batch,
                    int64_t rows, int64_t cols, int fmt, int block_along_rows, void* stream) {
  if (!x_bf16 || !codes || !scales_e8m0) return FSA_ERR_INVALID_ARG;
  if (batch <= 0 || rows <= 0 || cols <= 0) return FSA_ERR_INVALID_ARG;
  if (!fmt_ok(fmt)) return FSA_ERR_INVALID_ARG;
  if (block_along_rows != 0 && block_along_rows != 1) return FSA_ERR_INVALID_ARG;
  const int bits = fmt_bits(fmt);
  const int64_t valid = block_along_rows ? rows : cols;
  const int64_t out_rows = block_along_rows ? cols : rows;
  const int64_t nb = (valid + 31) / 32;
  if ((double)batch * out_rows * nb > 2147483647.0 * 256.0) return FSA_ERR_INVALID_ARG;
  if ((double)batch * rows * cols > 9.0e18) return FSA_ERR_INVALID_ARG;
  return quantize(static_cast<const uint16_t*>(x_bf16), static_cast<uint8_t*>(codes),
                  static_cast<uint8_t*>(scales_e8m0), batch, rows, cols, out_rows, nb,
                  nb * 4 * bits, nb, fmt, block_along_rows,
                  static_cast<hipStream_t>(stream));
}

int fsa_attention_fwd_ex(const void* q, const void* k, const void* v, void* out, int B, int H,
                         int S, int D, int fmt, int causal, const fsa_options* opt,
                         void* stream_) {
  int st = validate_attn(q, k, v, out, B, H, S, D, causal);
  if (st != FSA_OK) return st;
  const int* head_fmt = opt ? opt->head_fmt : nullptr;
  if (head_fmt) {
    for (int h = 0; h < H; ++h)
      if (!fmt_ok(head_fmt[h])) return FSA_ERR_INVALID_ARG;
  } else if (!fmt_ok(fmt)) {
    return FSA_ERR_INVALID_ARG;
  }
  hipStream_t stream = static_cast<hipStream_t>(stream_);

  // runs of consecutive heads with one format
  std::vector<RunLayout> runs;
  for (int h = 0; h < H;) {
    const int f = head_fmt ? head_fmt[h] : fmt;
    int e = h + 1;
    while (e < H && (head_fmt ? head_fmt[e] : fmt) == f) ++e;
    RunLayout rl{};
    rl.h0 = h;
    rl.hrun = e - h;
    rl.fmt = f;
    runs.push_back(rl);
    h = e;
  }

  const int64_t sk_alloc = round_up(S, kKeyTile);
  Carver cv;
  for (RunLayout& rl : runs) {
    const int bits = fmt_bits(rl.fmt);
    const int64_t nbh = (int64_t)B * rl.hrun;
    rl.kc = cv.take((size_t)(nbh * sk_alloc * D * bits / 8));
    rl.ks = cv.take((size_t)(nbh * sk_alloc * (D / 32)));
    rl.vc = cv.take((size_t)(nbh * D * sk_alloc * bits / 8));
    rl.vs = cv.take((size_t)(nbh * D * (sk_alloc / 32)));
  }
  // per-row frozen max and fallback offset, which the fallback pass reads
  // back; the caller's arrays when given
  const int64_t n_rows = (int64_t)B * H * S;
  const bool own_kappa = !(opt && opt->row_kappa);
  const bool own_mguess = !(opt && opt->row_max_guess);
  const size_t rk_off = own_kappa ? cv.take((size_t)n_rows * 4) : 0;
  const size_t rm_off = own_mguess ? cv.take((size_t)n_rows * 4) : 0;
  const size_t flag_off = cv.take(8);
  uint8_t* ws = nullptr;
  st = workspace(cv.off, &ws);
  if (st != FSA_OK) return st;
  int32_t* row_kappa = own_kappa ? reinterpret_cast<int32_t*>(ws + rk_off) : opt->row_kappa;
  float* row_mguess = own_mguess ? reinterpret_cast<float*>(ws + rm_off) : opt->row_max_guess;

  const uint16_t* qb = static_cast<const uint16_t*>(q);
  const uint16_t* kb = static_cast<const uint16_t*>(k);
  const uint16_t* vb = static_cast<const uint16_t*>(v);

  // MX-quantise K (blocks along D) and V (blocks along the keys, stored
  // transposed) for every run; padding rows and blocks get zero codes.  Q is
  // quantised inside the attention kernel, after scaling by the softmax scale
  // in binades, c = fp32(log2(e) / sqrt(D)), so that the score product comes
  // out in binades of the probability.
  const float score_scale = (float)((1.0 / std::log(2.0)) / std::sqrt((double)D));
  for (const RunLayout& rl : runs) {
    const int bits = fmt_bits(rl.fmt);
    const int64_t rb = (int64_t)D * bits / 8;
    for (int b = 0; b < B; ++b) {
      const int64_t src = ((int64_t)b * H + rl.h0) * S * D;
      const int64_t w0 = (int64_t)b * rl.hrun;
      st = quantize(kb + src, ws + rl.kc + w0 * sk_alloc * rb, ws + rl.ks + w0 * sk_alloc * (D / 32),
                    rl.hrun, S, D, sk_alloc, D / 32, rb, D / 32, rl.fmt, 0, stream, 1.0f,
                    fsa::SCALES_KEY_TILES);
      if (st != FSA_OK) return st;
      st = quantize(vb + src, ws + rl.vc + w0 * D * (sk_alloc * bits / 8),
                    ws + rl.vs + w0 * D * (sk_alloc / 32), rl.hrun, S, D, D, sk_alloc / 32,
                    sk_alloc * bits / 8, sk_alloc / 32, rl.fmt, 1, stream, 1.0f,
                    fsa::SCALES_DIM_TILES);
      if (st != FSA_OK) return st;
    }
  }
  if (opt && opt->event_after_quantize) {
    if (hipEventRecord(static_cast<hipEvent_t>(opt->event_after_quantize), stream) != hipSuccess)
      return FSA_ERR_HIP;
  }

  for (const RunLayout& rl : runs) {
    fsa::AttnArgs a;
    a.q = qb;
    a.qmul = score_scale;
    a.kc = ws + rl.kc; a.ks = ws + rl.ks;
    a.vc = ws + rl.vc; a.vs = ws + rl.vs;
    a.out = static_cast<uint16_t*>(out);
    a.row_kappa = row_kappa;
    a.row_mguess = row_mguess;
    a.B = B; a.H = H; a.S = S;
    a.h0 = rl.h0; a.hrun = rl.hrun;
    a.sk_alloc = (int)sk_alloc;
    a.bias = opt ? opt->guess_bias : 0.0f;
    a.fb_flag = reinterpret_cast<uint64_t*>(ws + flag_off);
    a.call_id = next_call_id();
    if (fsa::launch_fsa_fwd(a, kern_fmt(rl.fmt), D, causal, stream) != hipSuccess)
      return FSA_ERR_HIP;
  }
  return FSA_OK;
}

int fsa_attention_fwd(const void* q, const void* k, const void* v, void* out, int B, int H, int S,
                      int D, int fmt, int causal, void* stream) {
  return fsa_attention_fwd_ex(q, k, v, out, B, H, S, D, fmt, causal, nullptr, stream);
}

int fsa_attention_bf16_ref(const void* q, const void* k, const void* v, void* out, int B, int H,
                           int S, int D, int causal, void* stream) {
  const int st = validate_attn(q, k, v, out, B, H, S, D, causal);
  if (st != FSA_OK) return st;
  fsa::Bf16Args a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.out = static_cast<uint16_t*>(out);
  a.BH = B * H;
  a.S = S;
  a.s_alloc = (int)round_up(S, fsa::BF16_KEY_TILE);
  uint8_t* ws = nullptr;
  const int wst = workspace((size_t)a.BH * D * a.s_alloc * 2, &ws);
  if (wst != FSA_OK) return wst;
  a.vt = reinterpret_cast<uint16_t*>(ws);
  a.scale_log2 = (float)(1.0 / std::log(2.0) / std::sqrt((double)D));
  return fsa::launch_bf16_fa(a, D, causal, static_cast<hipStream_t>(stream)) == hipSuccess
             ? FSA_OK
             : FSA_ERR_HIP;
}

int fsa_debug_operands(const void* q, const void* k, const void* v, int B, int H, int S, int D,
                       int fmt, void* q_codes, void* q_scales, void* k_codes, void* k_scales,
                       void* v_codes, void* v_scales, void* stream_) {
  if (!q || !k || !v) return FSA_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || S <= 0 || D <= 0 || !fmt_ok(fmt)) return FSA_ERR_INVALID_ARG;
  if ((q_codes == nullptr) != (q_scales == nullptr) || (k_codes == nullptr) != (k_scales == nullptr) ||
      (v_codes == nullptr) != (v_scales == nullptr))
    return FSA_ERR_INVALID_ARG;
  if ((double)B * H * S * D > 1099511627776.0) return FSA_ERR_INVALID_ARG;
  for (const void* p : {q, k, v})
    if (reinterpret_cast<uintptr_t>(p) & 15) return FSA_ERR_INVALID_ARG;
  for (const void* p : {(const void*)q_codes, (const void*)k_codes, (const void*)v_codes})
    if (reinterpret_cast<uintptr_t>(p) & 15) return FSA_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return FSA_ERR_UNSUPPORTED;
  if (round_up(S, kKeyTile) * D * 2 >= ((int64_t)1 << 31)) return FSA_ERR_UNSUPPORTED;
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  const int bits = fmt_bits(fmt);
  const int64_t nbh = (int64_t)B * H;
  const int64_t sk = round_up(S, kKeyTile);
  const int64_t rb = (int64_t)D * bits / 8;
  if (q_codes) {
    fsa::QDumpArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.rows = nbh * S;
    a.qmul = (float)((1.0 / std::log(2.0)) / std::sqrt((double)D));
    a.codes = static_cast<uint8_t*>(q_codes);
    a.scales = static_cast<uint8_t*>(q_scales);
    if (fsa::launch_q_operand_dump(a, kern_fmt(fmt), D, stream) != hipSuccess) return FSA_ERR_HIP;
  }
  // the same quantiser calls as the attention path makes into its workspace
  if (k_codes) {
    const int st = quantize(static_cast<const uint16_t*>(k), static_cast<uint8_t*>(k_codes),
                            static_cast<uint8_t*>(k_scales), nbh, S, D, sk, D / 32, rb, D / 32, fmt, 0,
                            stream, 1.0f, fsa::SCALES_KEY_TILES);
    if (st != FSA_OK) return st;
  }
  if (v_codes) {
    const int st = quantize(static_cast<const uint16_t*>(v), static_cast<uint8_t*>(v_codes),
                            static_cast<uint8_t*>(v_scales), nbh, S, D, D, sk / 32, sk * bits / 8, sk / 32,
                            fmt, 1, stream, 1.0f, fsa::SCALES_DIM_TILES);
    if (st != FSA_OK) return st;
  }
  return FSA_OK;
}

int fsa_release_workspace(void) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FSA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  auto it = g_ws.find(dev);
  if (it == g_ws.end() || !it->second.ptr) return FSA_OK;
  if (hipFree(it->second.ptr) != hipSuccess) return FSA_ERR_HIP;
  it->second = Workspace();
  return FSA_OK;
}

}  // extern "C"
