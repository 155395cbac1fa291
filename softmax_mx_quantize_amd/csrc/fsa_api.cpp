// C ABI of the fused-softmax MX attention library: argument validation,
// per-device workspace, launch sequencing and error mapping.  Declarations
// and the contract of every entry point are in include/fsa.h.
#include "fsa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
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
// largest |fsa_options::guess_bias|, in binades.  The bias cancels out of
// the re-based sweep, but the first pass and the fallback pass's measure of
// a row's offset run from the biased reference: their fp32 score sums, about
// 2^23 (189 + |bias|) in magnitude, keep a spacing below 2^-12 binade up to
// this bound, far inside the rounding margins of the offset's binade.
constexpr float kMaxGuessBias = 1024.0f;

int fmt_bits(int fmt) { return fmt == FSA_MXFP8_E4M3 ? 8 : (fmt == FSA_MXFP6_E2M3 ? 6 : 4); }
bool fmt_ok(int fmt) { return fmt == FSA_MXFP8_E4M3 || fmt == FSA_MXFP6_E2M3 || fmt == FSA_MXFP4_E2M1; }

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// fsa_fmt -> kernel format index
int kern_fmt(int fmt) { return fmt == FSA_MXFP8_E4M3 ? 0 : (fmt == FSA_MXFP6_E2M3 ? 1 : 2); }

struct Workspace {
  void* ptr = nullptr;
  size_t bytes = 0;
  hipStream_t stream = nullptr;      // the stream of the last call that used it
};

std::mutex g_mu;

// Serialises the enqueue sequences of the calls that use a device's shared
// workspace or fixed scratch: from taking the buffer to the call's last
// launch no other call may enqueue work into it.  Calls from several host
// threads on one stream would otherwise interleave their kernels there (one
// call's quantiser overwriting operands another call's attention has yet to
// read).  Taken before g_mu, never after it.
std::mutex g_call_mu;
std::unordered_map<int, Workspace> g_ws;

// Returns a device buffer of at least `need` bytes for the current device,
// for work enqueued on `stream`.  Growing it is stream-ordered: the new
// buffer comes from hipMallocAsync on `stream`, and the old one is released
// with hipFreeAsync on the stream of the call that last used it, after that
// call's kernels (no device-wide synchronisation).
int workspace(size_t need, hipStream_t stream, uint8_t** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FSA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  Workspace& w = g_ws[dev];
  if (w.bytes < need) {
    const size_t sz = round_up((int64_t)need, 1 << 21);
    void* np = nullptr;
    if (hipMallocAsync(&np, sz, stream) != hipSuccess) {
      (void)hipGetLastError();
      return FSA_ERR_NO_MEMORY;
    }
    if (w.ptr && hipFreeAsync(w.ptr, w.stream) != hipSuccess) {
      (void)hipFreeAsync(np, stream);
      return FSA_ERR_HIP;
    }
    w.ptr = np;
    w.bytes = sz;
  }
  w.stream = stream;
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

// One quantiser launch over `batch` contiguous [rows][cols] inputs of one
// format; outputs are contiguous too (out_rows rows of nb_out blocks each).
int quantize(const uint16_t* x, uint8_t* codes, uint8_t* scales, int64_t batch, int64_t rows,
             int64_t cols, int64_t out_rows, int64_t nb_out, int fmt, int mode, hipStream_t stream,
             int scale_layout = fsa::SCALES_ROWS) {
  fsa::QuantArgs a{};
  a.x = x;
  a.codes = codes;
  a.scales = scales;
  a.batch = batch;
  a.rows = rows;
  a.cols = cols;
  a.out_rows = out_rows;
  a.nb_out = nb_out;
  a.code_slab = out_rows * nb_out * 4 * fmt_bits(fmt);
  a.x_sb = rows * cols;
  a.x_sh = 0;
  a.x_sr = cols;
  a.nh = 1;
  a.batch0 = 0;
  a.mult = 1.0f;
  a.scale_layout = scale_layout;
  a.fmt[0] = (uint8_t)kern_fmt(fmt);
  return fsa::launch_mx_quant(a, 1 << kern_fmt(fmt), mode, stream) == hipSuccess ? FSA_OK : FSA_ERR_HIP;
}

// ---- the attention call, shared by the allocating and the allocation-free
// entry points

// Element strides (batch entry, head, row) of the four tensors.
struct Strides {
  int64_t q[3], k[3], v[3], o[3];
};

// One launch group: batch entries [b0, b0 + nb) and heads [h0, h0 + n) of
// each, each head in its own format.
struct Piece {
  int b0, nb, h0, n;
};

struct Call {
  int pm = 0, px = 0;              // P~ variant (PM_*); P~ format (1 E4M3, 2 E3M2; 0 the operands')
  const uint16_t *q, *k, *v;
  uint16_t* out;
  int B, H, S, D, causal;
  int64_t sk_alloc;
  float score_scale;
  hipStream_t stream;
  const fsa_options* opt;
  Strides st;
  std::vector<int> fmt;            // per head
};

int piece_bits(const Call& c, const Piece& p) {
  int bits = 4;
  for (int h = p.h0; h < p.h0 + p.n; ++h) bits = std::max(bits, fmt_bits(c.fmt[h]));
  return bits;
}

int piece_fset(const Call& c, const Piece& p) {
  int fs = 0;
  for (int h = p.h0; h < p.h0 + p.n; ++h) fs |= 1 << kern_fmt(c.fmt[h]);
  return fs;
}

// Sub-allocation of one piece's quantised operands (slabs of the widest
// format present) and, when the caller gives no per-row arrays, its rows'
// kappa and frozen max.
struct PieceLayout {
  size_t kc, ks, vc, vs, rk, rm, nk;
  int64_t kc_slab, vc_slab;
};

PieceLayout carve_piece(Carver& cv, const Call& c, const Piece& p, bool own_rows, int bits = 0) {
  if (bits == 0) bits = piece_bits(c, p);
  const int64_t nbh = (int64_t)p.nb * p.n;
  PieceLayout l{};
  l.kc_slab = c.sk_alloc * c.D * bits / 8;
  l.vc_slab = (int64_t)c.D * c.sk_alloc * bits / 8;
  l.kc = cv.take((size_t)(nbh * l.kc_slab));
  l.ks = cv.take((size_t)(nbh * c.sk_alloc * (c.D / 32)));
  l.vc = cv.take((size_t)(nbh * l.vc_slab));
  l.vs = cv.take((size_t)(nbh * c.D * (c.sk_alloc / 32)));
  l.nk = cv.take((size_t)nbh * sizeof(uint64_t));
  if (own_rows) {
    l.rk = cv.take((size_t)nbh * c.S * 4);
    l.rm = cv.take((size_t)nbh * c.S * 4);
  }
  return l;
}

// MX-quantise K (blocks along D) and V (blocks along the keys, stored
// transposed) of a piece, each head in its own format, in one launch each;
// padding rows and blocks get zero codes.
int quantize_piece(const Call& c, const Piece& p, uint8_t* base, const PieceLayout& l) {
  fsa::QuantArgs a{};
  a.batch = (int64_t)p.nb * p.n;
  a.rows = c.S;
  a.cols = c.D;
  a.nh = p.n;
  a.mult = 1.0f;
  for (int j = 0; j < p.n; ++j) a.fmt[j] = (uint8_t)kern_fmt(c.fmt[p.h0 + j]);
  const int fset = piece_fset(c, p);
  // V first: its launch also clears each head's NaN-key slot, which K's
  // launch then lowers to the first key row holding NaN or Inf
  a.nan_key = reinterpret_cast<uint64_t*>(base + l.nk);
  // V: output rows are the D columns, blocks along the keys
  a.x = c.v + p.b0 * c.st.v[0] + p.h0 * c.st.v[1];
  a.x_sb = c.st.v[0]; a.x_sh = c.st.v[1]; a.x_sr = c.st.v[2];
  a.codes = base + l.vc;
  a.scales = base + l.vs;
  a.out_rows = c.D;
  a.nb_out = c.sk_alloc / 32;
  a.code_slab = l.vc_slab;
  a.scale_layout = fsa::SCALES_DIM_TILES;
  a.key8 = 0;
  a.nan_init = 1;                  // clears each head's NaN-key slot for K's launch
  if (fsa::launch_mx_quant(a, fset, 1, c.stream) != hipSuccess) return FSA_ERR_HIP;
  // K: output rows are keys (padded to sk_alloc), blocks along D
  a.x = c.k + p.b0 * c.st.k[0] + p.h0 * c.st.k[1];
  a.x_sb = c.st.k[0]; a.x_sh = c.st.k[1]; a.x_sr = c.st.k[2];
  a.codes = base + l.kc;
  a.scales = base + l.ks;
  a.out_rows = c.sk_alloc;
  a.nb_out = c.D / 32;
  a.code_slab = l.kc_slab;
  a.scale_layout = fsa::SCALES_KEY_TILES;
  a.key8 = c.px == 1;              // FP8 key order for E4M3 P~ only
  a.nan_init = 0;                  // rows with NaN/Inf blocks: atomic minimum
  if (fsa::launch_mx_quant(a, fset, 0, c.stream) != hipSuccess) return FSA_ERR_HIP;
  return FSA_OK;
}

// The fused kernel's two launches (sweep, then fallback pass) for a piece.
// Q and O are read and written in place (Q is quantised in the kernel,
// times log2(e)/sqrt(D), so that the score product comes out in binades of
// the probability).  Per-row kappa and frozen max: `whole` arrays span
// [B][H][S] (the caller's, or the workspace's); otherwise they are the
// piece's own (one batch entry, S rows per head from its first head).
int attend_piece(const Call& c, const Piece& p, uint8_t* base, const PieceLayout& l, int32_t* rk,
                 float* rm, bool whole, uint64_t* flag) {
  fsa::AttnArgs a{};
  a.q = c.q + p.b0 * c.st.q[0];
  a.out = c.out + p.b0 * c.st.o[0];
  a.q_sb = c.st.q[0]; a.q_sh = c.st.q[1]; a.q_ss = c.st.q[2];
  a.o_sb = c.st.o[0]; a.o_sh = c.st.o[1]; a.o_ss = c.st.o[2];
  a.qmul = c.score_scale;
  a.kc = base + l.kc; a.ks = base + l.ks;
  a.vc = base + l.vc; a.vs = base + l.vs;
  a.kc_slab = l.kc_slab; a.vc_slab = l.vc_slab;
  a.nan_key = reinterpret_cast<const uint64_t*>(base + l.nk);
  const int64_t boff = (int64_t)p.b0 * c.H;            // first head row of the piece's batch entries
  if (whole) {
    a.row_kappa = rk + boff * c.S;
    a.row_mguess = rm + boff * c.S;
    a.row_bh0 = 0;
  } else {
    if (p.nb != 1) return FSA_ERR_INVALID_ARG;         // piece rows cover one batch entry
    a.row_kappa = rk;
    a.row_mguess = rm;
    a.row_bh0 = p.h0;
  }
  a.B = p.nb; a.H = c.H; a.S = c.S;
  a.h0 = p.h0; a.hrun = p.n;
  a.sk_alloc = (int)c.sk_alloc;
  a.bias = c.opt ? c.opt->guess_bias : 0.0f;
  a.fb_flag = flag;
  a.call_id = next_call_id();
  a.skip_fallback = c.opt ? c.opt->skip_fallback_pass : 0;
  // formats per head, and the order workgroups take the heads in: the
  // formats interleaved, so that each XCD's contiguous share of the items
  // holds each format in proportion
  std::vector<int> by_fmt[3];
  for (int j = 0; j < p.n; ++j) {
    const int f = kern_fmt(c.fmt[p.h0 + j]);
    a.hfmt[j] = (uint8_t)f;
    by_fmt[f].push_back(j);
  }
  {
    size_t at[3] = {0, 0, 0};
    int slot = 0;
    while (slot < p.n) {
      // take next from the format that is furthest behind its share
      int best = -1;
      double lag = 0.0;
      for (int f = 0; f < 3; ++f) {
        if (at[f] >= by_fmt[f].size()) continue;
        const double want = (double)(slot + 1) * by_fmt[f].size() / p.n - (double)at[f];
        if (best < 0 || want > lag) { best = f; lag = want; }
      }
      a.horder[slot++] = (uint8_t)by_fmt[best][at[best]++];
    }
  }
  return fsa::launch_fsa_fwd(a, piece_fset(c, p), c.pm, c.px, c.D, c.causal, c.stream) == hipSuccess
             ? FSA_OK
             : FSA_ERR_HIP;
}

int record_event(const Call& c) {
  if (c.opt && c.opt->event_after_quantize &&
      hipEventRecord(static_cast<hipEvent_t>(c.opt->event_after_quantize), c.stream) != hipSuccess)
    return FSA_ERR_HIP;
  return FSA_OK;
}

// Fixed scratch of the allocation-free entry point: one copy per device
// (each device that runs it holds it until the process ends).  In host code
// `scratch` names a host-side stand-in; its device address on each device
// comes from hipGetSymbolAddress, taken once per device with that device
// current, and only that address is handed to kernels.
constexpr size_t kScratchBytes = (size_t)64 << 20;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::unordered_map<int, uint8_t*> g_scratch;

int scratch_address(uint8_t** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FSA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch.find(dev);
  if (it == g_scratch.end()) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return FSA_ERR_HIP;
    }
    it = g_scratch.emplace(dev, static_cast<uint8_t*>(p)).first;
  }
  *out = it->second;
  return FSA_OK;
}

// Strides of a tensor argument: the caller's, or those of a contiguous
// [B][H][S][D] tensor.  Rows must start 16 bytes apart multiples (the
// kernels load 16-byte vectors); D is contiguous.
bool take_strides(const int64_t* given, int H, int S, int D, int64_t out[3]) {
  if (!given) {
    out[0] = (int64_t)H * S * D;
    out[1] = (int64_t)S * D;
    out[2] = D;
    return true;
  }
  for (int i = 0; i < 3; ++i) {
    if (given[i] < 0 || given[i] % 8 != 0) return false;
    out[i] = given[i];
  }
  return out[2] >= D;
}

int attention(const void* q, const void* k, const void* v, void* out, int B, int H, int S, int D,
              int fmt, int causal, const fsa_options* opt, void* stream_, bool no_alloc) {
  int st = validate_attn(q, k, v, out, B, H, S, D, causal);
  if (st != FSA_OK) return st;
  const int* head_fmt = opt ? opt->head_fmt : nullptr;
  if (head_fmt) {
    for (int h = 0; h < H; ++h)
      if (!fmt_ok(head_fmt[h])) return FSA_ERR_INVALID_ARG;
  } else if (!fmt_ok(fmt)) {
    return FSA_ERR_INVALID_ARG;
  }
  if (opt && (opt->row_kappa == nullptr) != (opt->row_max_guess == nullptr)) return FSA_ERR_INVALID_ARG;
  if (opt && !(std::fabs(opt->guess_bias) <= kMaxGuessBias)) return FSA_ERR_INVALID_ARG;
  const bool own_rows = !(opt && opt->row_kappa);

  Call c;
  c.q = static_cast<const uint16_t*>(q);
  c.k = static_cast<const uint16_t*>(k);
  c.v = static_cast<const uint16_t*>(v);
  c.out = static_cast<uint16_t*>(out);
  c.B = B; c.H = H; c.S = S; c.D = D; c.causal = causal;
  c.sk_alloc = round_up(S, kKeyTile);
  c.score_scale = (float)((1.0 / std::log(2.0)) / std::sqrt((double)D));
  c.stream = static_cast<hipStream_t>(stream_);
  c.opt = opt;
  const fsa_layout* lay = opt ? opt->layout : nullptr;
  if (!take_strides(lay ? lay->q : nullptr, H, S, D, c.st.q) ||
      !take_strides(lay ? lay->k : nullptr, H, S, D, c.st.k) ||
      !take_strides(lay ? lay->v : nullptr, H, S, D, c.st.v) ||
      !take_strides(lay ? lay->out : nullptr, H, S, D, c.st.o))
    return FSA_ERR_INVALID_ARG;
  c.fmt.assign(H, fmt);
  if (head_fmt) c.fmt.assign(head_fmt, head_fmt + H);
  // the P~ variant and the formats it needs
  const int pv = opt ? opt->p_variant : FSA_P_BLOCK;
  auto all_fmt = [&](std::initializer_list<int> ok) {
    for (int f : c.fmt)
      if (std::find(ok.begin(), ok.end(), f) == ok.end()) return false;
    return true;
  };
  switch (pv) {
    case FSA_P_BLOCK: break;
    case FSA_P_ROW_SCALE:
      if (!all_fmt({FSA_MXFP8_E4M3})) return FSA_ERR_UNSUPPORTED;
      c.pm = 1;
      break;
    case FSA_P_E4M3:
      if (!all_fmt({FSA_MXFP6_E2M3, FSA_MXFP4_E2M1})) return FSA_ERR_UNSUPPORTED;
      c.px = 1;
      break;
    case FSA_P_E3M2:
      if (!all_fmt({FSA_MXFP6_E2M3})) return FSA_ERR_UNSUPPORTED;
      c.px = 2;
      break;
    case FSA_P_AFFINE:
      if (!all_fmt({FSA_MXFP4_E2M1})) return FSA_ERR_UNSUPPORTED;
      c.pm = 2;
      break;
    case FSA_P_EXACT_EXP:
      // built for single formats and the FP6/FP4 hybrid
      if (!all_fmt({FSA_MXFP8_E4M3}) && !all_fmt({FSA_MXFP6_E2M3, FSA_MXFP4_E2M1}))
        return FSA_ERR_UNSUPPORTED;
      c.pm = 3;
      break;
    default: return FSA_ERR_INVALID_ARG;
  }

  std::lock_guard<std::mutex> call_lock(g_call_mu);
  if (!no_alloc) {
    // every batch entry and up to MAX_HEAD_TABLE heads per piece, side by
    // side in the growing workspace: quantise everything, then attend (the
    // event between the two marks the attention kernels)
    std::vector<Piece> pieces;
    for (int h = 0; h < H; h += fsa::MAX_HEAD_TABLE)
      pieces.push_back(Piece{0, B, h, std::min(fsa::MAX_HEAD_TABLE, H - h)});
    Carver cv;
    std::vector<PieceLayout> lays;
    for (const Piece& p : pieces) lays.push_back(carve_piece(cv, c, p, false));
    const size_t rk = own_rows ? cv.take((size_t)B * H * S * 4) : 0;
    const size_t rm = own_rows ? cv.take((size_t)B * H * S * 4) : 0;
    const size_t flag_off = cv.take(8);
    uint8_t* ws = nullptr;
    st = workspace(cv.off, c.stream, &ws);
    if (st != FSA_OK) return st;
    for (size_t i = 0; i < pieces.size(); ++i)
      if ((st = quantize_piece(c, pieces[i], ws, lays[i])) != FSA_OK) return st;
    if ((st = record_event(c)) != FSA_OK) return st;
    int32_t* rkp = own_rows ? reinterpret_cast<int32_t*>(ws + rk) : opt->row_kappa;
    float* rmp = own_rows ? reinterpret_cast<float*>(ws + rm) : opt->row_max_guess;
    for (size_t i = 0; i < pieces.size(); ++i) {
      st = attend_piece(c, pieces[i], ws, lays[i], rkp, rmp, true, reinterpret_cast<uint64_t*>(ws + flag_off));
      if (st != FSA_OK) return st;
    }
    return FSA_OK;
  }

  // allocation-free: pieces of one batch entry and as many heads as the
  // fixed scratch holds, each quantised and attended in turn (stream order
  // keeps a piece's reuse of the scratch behind the previous piece's
  // kernels)
  uint8_t* base = nullptr;
  if ((st = scratch_address(&base)) != FSA_OK) return st;
  // as many heads per piece as fit at the widest format of the call
  int n_fit = 0;
  for (int n = std::min(H, fsa::MAX_HEAD_TABLE); n >= 1; --n) {
    Carver cv;
    carve_piece(cv, c, Piece{0, 1, 0, n}, own_rows, piece_bits(c, Piece{0, 1, 0, H}));
    cv.take(8);
    if (cv.off <= kScratchBytes) { n_fit = n; break; }
  }
  if (n_fit == 0) return FSA_ERR_TOO_LARGE;          // one head does not fit
  bool event_done = false;
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; h += n_fit) {
      const Piece p{b, 1, h, std::min(n_fit, H - h)};
      Carver cv;
      const PieceLayout l = carve_piece(cv, c, p, own_rows);
      const size_t flag_off = cv.take(8);
      if (cv.off > kScratchBytes) return FSA_ERR_TOO_LARGE;
      if ((st = quantize_piece(c, p, base, l)) != FSA_OK) return st;
      if (!event_done) {
        if ((st = record_event(c)) != FSA_OK) return st;
        event_done = true;
      }
      if (own_rows)
        st = attend_piece(c, p, base, l, reinterpret_cast<int32_t*>(base + l.rk),
                          reinterpret_cast<float*>(base + l.rm), false,
                          reinterpret_cast<uint64_t*>(base + flag_off));
      else
        st = attend_piece(c, p, base, l, opt->row_kappa, opt->row_max_guess, true,
                          reinterpret_cast<uint64_t*>(base + flag_off));
      if (st != FSA_OK) return st;
    }
  return FSA_OK;
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
    case FSA_ERR_TOO_LARGE: return "one head exceeds the fixed 64 MiB scratch of the allocation-free call";
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
                  static_cast<uint8_t*>(scales_e8m0), batch, rows, cols, out_rows, nb, fmt,
                  block_along_rows, static_cast<hipStream_t>(stream));
}

int fsa_attention_fwd_ex(const void* q, const void* k, const void* v, void* out, int B, int H,
                         int S, int D, int fmt, int causal, const fsa_options* opt,
                         void* stream_) {
  return attention(q, k, v, out, B, H, S, D, fmt, causal, opt, stream_, false);
}

int fsa_attention_fwd_noalloc(const void* q, const void* k, const void* v, void* out, int B, int H,
                              int S, int D, int fmt, int causal, const fsa_options* opt,
                              void* stream_) {
  return attention(q, k, v, out, B, H, S, D, fmt, causal, opt, stream_, true);
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
  std::lock_guard<std::mutex> call_lock(g_call_mu);
  const int wst = workspace((size_t)a.BH * D * a.s_alloc * 2, static_cast<hipStream_t>(stream), &ws);
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
                            static_cast<uint8_t*>(k_scales), nbh, S, D, sk, D / 32, fmt, 0, stream,
                            fsa::SCALES_KEY_TILES);
    if (st != FSA_OK) return st;
  }
  if (v_codes) {
    const int st = quantize(static_cast<const uint16_t*>(v), static_cast<uint8_t*>(v_codes),
                            static_cast<uint8_t*>(v_scales), nbh, S, D, D, sk / 32, fmt, 1, stream,
                            fsa::SCALES_DIM_TILES);
    if (st != FSA_OK) return st;
  }
  return FSA_OK;
}

int fsa_release_workspace(void) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FSA_ERR_HIP;
  std::lock_guard<std::mutex> call_lock(g_call_mu);
  std::lock_guard<std::mutex> lock(g_mu);
  auto it = g_ws.find(dev);
  if (it == g_ws.end() || !it->second.ptr) return FSA_OK;
  // after the last call's kernels on its stream; the caller has finished
  // with every call (documented), so waiting on that stream suffices
  if (hipFreeAsync(it->second.ptr, it->second.stream) != hipSuccess) return FSA_ERR_HIP;
  if (hipStreamSynchronize(it->second.stream) != hipSuccess) return FSA_ERR_HIP;
  it->second = Workspace();
  return FSA_OK;
}

}  // extern "C"
