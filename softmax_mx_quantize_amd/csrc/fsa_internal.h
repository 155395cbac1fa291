// Host-visible launch interfaces between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fsa {

// MX quantiser geometry.  MODE 0: blocks along `cols`; output row o in
// [0, batch*out_rows) maps to input row o % out_rows (rows >= `rows` are
// padding and get zero codes and scale byte 0).  MODE 1: blocks along
// `rows`, output row o in [0, batch*cols) is input column o % cols
// (out_rows must equal cols).  Blocks b >= ceil(valid/32) up to nb_out are
// zero padding.
struct QuantArgs {
  const uint16_t* x;
  uint8_t* codes;
  uint8_t* scales;
  int64_t batch, rows, cols;
  int64_t out_rows;      // output rows per batch
  int64_t nb_out;        // blocks per output row
  int64_t code_stride;   // bytes between output code rows
  int64_t scale_stride;  // bytes between output scale rows
  int64_t batch0;        // first batch entry of this launch (columns mode)
  float mult;            // every input value is multiplied by this (fp32) first
  int scale_layout;      // SCALES_* below
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

hipError_t launch_mx_quant(const QuantArgs& a, int fmt, int mode, hipStream_t stream);

// Fused attention for the heads [h0, h0+hrun) of every batch entry.  Q is
// read as bf16 and MX-quantised in the kernel (times qmul); K^ and V^ come
// from the quantiser.  Workspace slabs are indexed by w = b*hrun + (h - h0):
//   K^ codes [BH][sk_alloc][D*bits/8], scales in the KEY_TILES layout
//   V^ (transposed) codes [BH][D][sk_alloc*bits/8], scales in DIM_TILES
// sk_alloc covers every key tile; the padding holds zero codes.
struct AttnArgs {
  const uint16_t* q;             // bf16 [B][H][S][D]
  const uint8_t* kc; const uint8_t* ks;
  const uint8_t* vc; const uint8_t* vs;
  uint16_t* out;                 // bf16 [B][H][S][D]
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
};

hipError_t launch_fsa_fwd(const AttnArgs& a, int fmt, int D, int causal, hipStream_t stream);

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
