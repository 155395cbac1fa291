// Host-visible launch interfaces between the C ABI layer and the kernels.
#pragma once

#include <cstddef>

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fsa {

// Heads of one launch whose formats and order travel in the kernel
// arguments (at most this many per launch).
constexpr int MAX_HEAD_TABLE = 256;

// MX quantiser geometry.  The launch covers `batch` slabs; slab w reads head
// w % nh of batch entry w / nh: element (r, c) at x + (w / nh) * x_sb +
// (w % nh) * x_sh + r * x_sr + c (columns contiguous).  MODE 0: blocks along
// `cols`, output row r of slab w is input row r (rows >= `rows` are padding:
// zero codes, scale byte 0).  MODE 1: blocks along `rows`, output row r of
// slab w is input column r (out_rows must equal cols).  Blocks
// b >= ceil(valid/32) up to nb_out are zero padding.  A code row takes
// nb_out * 4 * bits bytes (bits of the slab's format), a slab's codes start
// at w * code_slab; scale rows take nb_out bytes, out_rows of them per slab.
struct QuantArgs {
  const uint16_t* x;
  uint8_t* codes;
  uint8_t* scales;
  int64_t batch, rows, cols;
  int64_t out_rows;      // output rows per slab
  int64_t nb_out;        // blocks per output row
  int64_t code_slab;     // bytes between slabs' codes
  int64_t x_sb, x_sh, x_sr;   // input element strides
  int nh;                // heads per batch entry
  int64_t batch0;        // first slab of this launch (columns mode)
  float mult;            // every input value is multiplied by this (fp32) first
  int scale_layout;      // SCALES_* below
  int key8;              // KEY_TILES in the FP8 key order whatever the codes (E4M3 P~)
  // Per slab, the first row of a block holding NaN or Inf (the attention
  // path's K^: every score against that key is NaN).  Rows mode: atomic
  // minimum of the row over such blocks; columns mode with nan_init: set to
  // all ones first (the call launches V's quantiser before K's).  Null: off.
  uint64_t* nan_key;
  int nan_init;
  uint8_t fmt[MAX_HEAD_TABLE];  // element format (FMT_*) of head slot w % nh
};

// Scale byte layouts.  ROWS: scales[row][block] (the public layout).  The two
// tile layouts feed the attention kernel (32x32x64 scaled MFMA, D a multiple
// of 64): per 128-key tile, lane (h, rho) = 32 h + rho of that product finds
// the bytes of its products next to each other (NB = D/16 bytes for K^ and
// for V^T, at lane * NB), so one LDS read fetches them and the MFMA picks its
// byte with op_sel.
enum { SCALES_ROWS = 0, SCALES_KEY_TILES = 1, SCALES_DIM_TILES = 2 };

// Byte of key row Rl (0..127 within its tile) and D block blk in a KEY_TILES
// tile of 128 * D/32 bytes.  The score product covers 64-key chunk u = Rl / 64
// with two 32-row blocks b; its A row rho = 8 j + 4 x + k holds key
// 32 x + 16 b + 4 j + k of the chunk (FP6/FP4) or 32 b + 16 x + 4 j + k (FP8),
// so that a lane's 32 outputs are the keys it supplies to the P V product.
// Lane half h reads D block 2 c + h of 64-wide D chunk c; its byte for
// (u, b, c) is u*2nd + b*nd + c.
__host__ __device__ inline int key_tile_byte(int rl, int blk, int d, int bits) {
  const int nd = d / 64;
  const int u = rl >> 6, kk = rl & 63;
  const int hi = kk >> 5, mid = (kk >> 4) & 1, j = (kk >> 2) & 3, k = kk & 3;
  const int x = bits == 8 ? mid : hi, b = bits == 8 ? hi : mid;
  const int rho = 8 * j + 4 * x + k;
  return (32 * (blk & 1) + rho) * 4 * nd + u * 2 * nd + b * nd + (blk >> 1);
}
// Byte of output row dd (0..D-1) and key block kb (0..3 within its tile) in a
// DIM_TILES tile of 4 D bytes: the P V product's A row rho = dd % 32 of
// 32-row block db = dd / 32, lane half h = kb % 2 of 64-key chunk u = kb / 2.
__host__ __device__ inline int dim_tile_byte(int dd, int kb, int d) {
  return (32 * (kb & 1) + (dd & 31)) * (d / 16) + (kb >> 1) * (d / 32) + (dd >> 5);
}

// `fset`: the formats present in a.fmt[0, nh), as a bit set (1 << FMT_*).
hipError_t launch_mx_quant(const QuantArgs& a, int fset, int mode, hipStream_t stream);

// Fused attention for the heads [h0, h0+hrun) of every batch entry, head
// h0 + j in element format hfmt[j].  Q is read as bf16 and MX-quantised in
// the kernel (times qmul); K^ and V^ come from the quantiser.  Workspace
// slabs are indexed by w = b*hrun + j, kc_slab / vc_slab bytes apart (the
// widest format's size), each packed in its head's own format:
//   K^ codes [sk_alloc][D*bits/8], scales [sk_alloc][D/32] in the KEY_TILES
//   layout; V^ (transposed) codes [D][sk_alloc*bits/8], scales in DIM_TILES.
// sk_alloc covers every key tile; the padding holds zero codes.  Q and O
// element (b, h, s, d) sit at b*sb + h*sh + s*ss + d.
struct AttnArgs {
  const uint16_t* q;             // bf16
  const uint8_t* kc; const uint8_t* ks;
  const uint8_t* vc; const uint8_t* vs;
  uint16_t* out;                 // bf16
  int64_t q_sb, q_sh, q_ss;      // element strides of Q
  int64_t o_sb, o_sh, o_ss;      // element strides of O
  int64_t kc_slab, vc_slab;      // bytes between K^ / V^T code slabs
  int32_t* row_kappa;            // rows of heads bh >= row_bh0 (bh = b*H + h), S per head:
  float* row_mguess;             //   kappa and frozen max (binades), written by the first
  int64_t row_bh0;               //   pass and read by the fallback pass
  int B, H, S;
  int h0, hrun;                  // heads [h0, h0+hrun) of each batch entry
  int sk_alloc;
  float qmul;                    // log2(e) / sqrt(D), applied to Q before quantisation
  float bias;                    // added to every frozen max, binades
  uint64_t* fb_flag;             // stamped with call_id when a row needs the fallback
  uint64_t call_id;              // unique per call (never 0)
  int skip_fallback;             // 1: no fallback-pass launch (rows beyond EXT stay wrong)
  const uint64_t* nan_key;       // per slab: first key row with a NaN/Inf K^ block (~0: none)
  uint8_t hfmt[MAX_HEAD_TABLE];  // element format (FMT_*) of head h0 + j
  uint8_t horder[MAX_HEAD_TABLE];  // head slot -> j: the order workgroups take heads in
};
// the kernel reads both byte tables a dword at a time
static_assert(offsetof(AttnArgs, hfmt) % 4 == 0 && offsetof(AttnArgs, horder) % 4 == 0 &&
                  MAX_HEAD_TABLE % 4 == 0,
              "byte tables must be dword-aligned");

// LDS stages of the attention kernel (128-byte rows): one 128-key tile of
// K^ rows plus its scales, and D rows of V^T plus theirs.
constexpr int attn_kstage_bytes(int d) { return 128 * 128 + 128 * (d / 32); }
constexpr int attn_vstage_bytes(int d) { return d * 128 + 4 * d; }

// `fset`: the formats present in a.hfmt[0, hrun), as a bit set (1 << FMT_*);
// `pm` the P~ variant (PM_* of fsa_common.h: 0 block scales, 1 one scale
// per row, 2 affine E2M1 codes, 3 exact exponential); `px` the P~ format
// when it differs from the operands' (1 E4M3 over FP6/FP4, 2 E3M2 over
// E2M3).  hipErrorInvalidValue for a combination that is not built.
hipError_t launch_fsa_fwd(const AttnArgs& a, int fset, int pm, int px, int D, int causal,
                          hipStream_t stream);

// The attention kernel's Q' operands written out (a debug view): rows of
// bf16 Q [rows][D] times qmul, MX-quantised by the very device functions of
// the kernel's prologue.  codes [rows][D*bits/8] in the public packing,
// scales [rows][D/32]: each block's E8M0 byte raised by 23 as the score
// product consumes it (2^23 rides on Q's scale; 254 at most, 255 for NaN).
struct QDumpArgs {
  const uint16_t* q;
  int64_t rows;
  float qmul;
  uint8_t* codes;
  uint8_t* scales;
};

hipError_t launch_q_operand_dump(const QDumpArgs& a, int fmt, int D, hipStream_t stream);

// Plain BF16 flash attention.
constexpr int BF16_KEY_TILE = 64;
struct Bf16Args {
  const uint16_t* q; const uint16_t* k; const uint16_t* v;
  uint16_t* out;
  uint16_t* vt;                  // workspace: V^T [BH][D][s_alloc]
  int BH, S;
  int s_alloc;                   // S rounded up to BF16_KEY_TILE
  float scale_log2;              // log2(e) / sqrt(D)
};

hipError_t launch_bf16_fa(const Bf16Args& a, int D, int causal, hipStream_t stream);

}  // namespace fsa
