// Internal interface between the host driver (rmt_lib.hip) and the gfx950
// kernels.  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace rmt {

// Largest number of cells one grouped launch covers.  The per-group table
// travels by value in the kernel arguments, so nothing about a diagonal is
// stored in device memory.
constexpr int kMaxGroups = 32;

// Per-launch group table.  Group g is one (layer, segment) cell of the
// current diagonal; its R rows are split in two ranges that may live in
// different buffers: rows [0, split) at *_lo[g], rows [split, R) at *_hi[g]
// (the split points are launch arguments).  This is how a cell reads
// [M(l, s-1); X(l-1, s)] and writes X(l, s) and M(l, s) without copies.
struct GroupTable {
  int32_t G;
  int32_t layer[kMaxGroups];
  const void* in_lo[kMaxGroups];
  const void* in_hi[kMaxGroups];
  void* out_lo[kMaxGroups];
  void* out_hi[kMaxGroups];
};

// Side outputs that prepare the next RMSNorm (the residual epilogues, the
// segment gather and the memory preparation write them): for output row y of
// group g -- split like out_lo / out_hi -- the bf16 copy y * gamma[layer] and
// the sums of y^2 over each 64-column chunk of the row (N / 64 floats per
// row, each summed in one fixed order).  The consumer reduces the chunks in
// order to 1 / sqrt(mean(y^2) + eps) and scales its GEMM rows by it.  Every
// pointer must be valid (rows nobody reads go to a discard area).
// The chunk sums are stored chunk-major, ss[j * ss_ld + r] for row r and
// chunk j, so that a wave's sums for 32 consecutive rows of one chunk fill
// whole 128-byte lines (row-major, the 4-byte sums of one row would come
// from as many workgroups as the row has chunks, each leaving its line
// partly written).
constexpr int kChunk = 64;
struct NormAux {
  void* rows_lo[kMaxGroups];       // 16-bit [rows][N]
  void* rows_hi[kMaxGroups];
  float* ss_lo[kMaxGroups];        // fp32 [N / kChunk][ss_ld_lo]
  float* ss_hi[kMaxGroups];        // fp32 [N / kChunk][ss_ld_hi]
  int32_t layer_lo[kMaxGroups];    // gain row for the lo / hi rows
  int32_t layer_hi[kMaxGroups];
  int32_t ss_ld_lo, ss_ld_hi;      // row capacity of the lo / hi sum regions
};

enum GemmEpilogue : int {
  EPI_STORE_BF16 = 0,  // C = bf16(acc)
  EPI_QKV_ROPE = 1,    // C = bf16(rope(acc)) on Q/K columns, bf16(acc) on V
  EPI_SWIGLU = 2,      // gate/up interleaved in 32-column blocks: U = silu(g) * u
  EPI_RESID_F32 = 3,   // C = acc + residual, fp32, split row destinations
  EPI_BIAS_BF16 = 4,        // C = bf16(acc + bias)
  EPI_BIAS_RELU_BF16 = 5,   // C = bf16(max(acc + bias, 0))
  EPI_RESID_BIAS_F32 = 6,   // C = residual + (acc + bias), fp32, split row destinations
  EPI_RESID_NORM_F32 = 7,   // EPI_RESID_F32 plus the NormAux side outputs of the rows
};

struct GemmArgs {
  const uint16_t* A;   // bf16 rows [G*M][K] (group g owns rows g*M .. g*M+M-1)
  const uint16_t* B;   // bf16 [Lw][N][K]: B_l stored transposed, K contiguous
  int M, N, K;
  int split_in;        // residual rows: [0, split_in) from in_lo, rest from in_hi
  int split_out;       // output rows: [0, split_out) to out_lo, rest to out_hi
  int ld_res;          // residual row stride (elements)
  int ld_out;          // output row stride (elements)
  const float2* rope;  // EPI_QKV_ROPE: (cos, sin) table [M][hd/2]
  int rope_cols;       // EPI_QKV_ROPE: columns [0, rope_cols) are rotated, in 64-column
                       //   groups whose column c < 32 pairs with c + 32, at frequency index
                       //   32 ((col % hd) / 64) + col % 32 (PACK_ROPE_PAIRS order for hd 128)
  int hd;              // EPI_QKV_ROPE: head dimension (64 or 128)
  const float* bias;   // EPI_*BIAS*: fp32 [Lw][N], row layer[g] added to every output row
  int q_cols;          // EPI_QKV_ROPE, EPI_BIAS_BF16: columns [0, q_cols) (a multiple of 32)
  float q_scale;       //   are multiplied by q_scale before the bf16 rounding (0 cols: none)
  int f16;             // 1: A, B and 16-bit results are fp16 instead of bf16 (EPI_STORE_BF16,
                       //    EPI_QKV_ROPE, EPI_SWIGLU, EPI_RESID_F32 only)
  int a_split;         // EPI_QKV_ROPE: > 0: A rows [0, a_split) of group g from tab.in_lo[g],
                       //   rows from a_split on from tab.in_hi[g] (16-bit rows of K; a
                       //   multiple of 8); 0: A packed per group as above
  const float* row_scale;  // EPI_QKV_ROPE, EPI_SWIGLU: non-null: output row r of group g is
                           //   multiplied by row_scale[g * M + r] first (an RMSNorm's 1/rms)
  const float* aux_gamma;  // EPI_RESID_NORM_F32: gains [Lw][N] of the side outputs
};

// Softmax scale of attention in the base-2 domain, log2(e) / sqrt(hd).  The
// QKV projection folds it into Q for the attention stage of the model, so
// both sides must use this one value.
inline float attention_scale_log2(int hd) { return 1.4426950408889634f / sqrtf((float)hd); }

hipError_t launch_gemm(int epilogue, const GemmArgs& a, const GroupTable& tab, hipStream_t stream,
                       const NormAux* aux = nullptr);

// 1 / sqrt(sum of a row's chunk sums / d + eps) for every row of every group
// (rows [0, split) from ss_lo[g], the rest from ss_hi[g] of `aux`), packed
// into rinv [G * R].
hipError_t launch_row_rinv(int G, int R, int d, int split, const NormAux& aux, float eps, float* rinv,
                           hipStream_t stream);
// Side outputs for fp32 rows that no GEMM epilogue produced: `rows` rows of
// `src` [rows][d] in regions of rows_per_layer rows; region q uses gain row
// layer0 + q % L.  Writes the 16-bit copy dst16 [rows][d] (bf16, or fp16 per
// f16) and the chunk sums, chunk-major per region: dss + q * rows_per_layer *
// (d / 64) holds [d / 64][rows_per_layer].
hipError_t launch_norm_aux_rows(int rows, int d, const float* src, int rows_per_layer, int L,
                                int layer0, const float* gamma, uint16_t* dst16, float* dss,
                                bool f16, hipStream_t stream);

// Row-wise RMSNorm of every group's R rows (fp32 in, bf16 -- or fp16 when
// f16 is set -- out, packed).
hipError_t launch_rmsnorm(int G, int R, int d, int split_in, const GroupTable& tab,
                          const float* gamma, float eps, uint16_t* out, hipStream_t stream,
                          bool f16 = false);
// Row-wise LayerNorm (gain gamma, shift beta, both [Lw][d]), same layout.
hipError_t launch_layernorm(int G, int R, int d, int split_in, const GroupTable& tab,
                            const float* gamma, const float* beta, float eps, uint16_t* out,
                            hipStream_t stream);
// LayerNorm with an fp32 result written to out_lo[g] (rows < split_out) or
// out_hi[g], and also the packed bf16 copy when out_bf16 is not null.
hipError_t launch_layernorm_f32(int G, int R, int d, int split_in, int split_out,
                                const GroupTable& tab, const float* gamma, const float* beta,
                                float eps, uint16_t* out_bf16, hipStream_t stream);
// Rows of every group as bf16, packed (no normalisation).
hipError_t launch_cast_rows(int G, int R, int d, int split_in, const GroupTable& tab, uint16_t* out,
                            hipStream_t stream);

// X(-1, s) rows -> fp32 slot: token-id lookup (bf16 table) or a row copy.
// With dst16 non-null the lookup also writes the RMSNorm side outputs of the
// rows (gain row `gamma`, [d]): dst16 [n][d] and the chunk sums dss
// [d / 64][ss_ld] (chunk-major, ss_ld >= n).
hipError_t launch_gather_tokens(int n, int d, const int32_t* ids, int V, const uint16_t* embed,
                                float* dst, int32_t* bad_flag, hipStream_t stream,
                                const float* gamma = nullptr, uint16_t* dst16 = nullptr,
                                float* dss = nullptr, int ss_ld = 0, bool f16 = false);
hipError_t launch_copy_rows_bf16(int n, int d, const uint16_t* src, float* dst,
                                 hipStream_t stream);

// Attention over each group's R rows, causal or unmasked; Hq / Hkv must be
// 1, 2 or a multiple of 4.  q_prescaled: Q already carries the softmax scale
// attention_scale_log2(hd) (the QKV epilogue applied it).  f16: Q/K/V, the
// probabilities and the output are fp16 instead of bf16 (causal, prescaled
// only: the LLaMA-shaped cell).
hipError_t launch_attention(const uint16_t* qkv, uint16_t* out, int G, int R, int Hq, int Hkv,
                            int hd, bool causal, bool q_prescaled, hipStream_t stream,
                            bool f16 = false);

// fp32 linear + bias + GELU cell with the split write-back.
hipError_t launch_linear_gelu_f32(int G, int R, int d, int split_in, int split_out,
                                  const GroupTable& tab, const float* W, const float* bias,
                                  hipStream_t stream);

// Weight packing: dst[l][r][k] = src_sel(r)[l][k][col(r)] as bf16, or as fp16
// when dst_f16 is set (from fp32 or bf16, rounded to nearest even).
// PACK_PLAIN:      dst row r <- src0 column r (N_dst = N_src).
// PACK_GATE_UP:    dst row r in block r/64: first 32 rows <- src0 columns,
//                  last 32 rows <- src1 columns (N_dst = 2 N_src).
// PACK_ROPE_PAIRS: as PACK_PLAIN, except that the first pair_cols rows (a
//                  multiple of 128: the Q and K heads of 128) are reordered
//                  within each head into two 64-row groups, group q holding
//                  the dimensions 32 q .. 32 q + 31 and then 64 + 32 q ..
//                  64 + 32 q + 31: every rotation pair of RoPE (d, d + 64)
//                  then sits 32 rows apart inside one group, as it does in a
//                  64-wide head.  Q and K take the same order, so their dot
//                  products, and the attention, are unchanged.
enum PackMode : int { PACK_PLAIN = 0, PACK_GATE_UP = 1, PACK_ROPE_PAIRS = 2 };
hipError_t launch_pack(int L, int K, int N_src, const void* src0, const void* src1,
                       int src_is_bf16, int mode, uint16_t* dst, hipStream_t stream,
                       int dst_f16 = 0, int pair_cols = 0);

}  // namespace rmt
