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

enum GemmEpilogue : int {
  EPI_STORE_BF16 = 0,  // C = bf16(acc)
  EPI_QKV_ROPE = 1,    // C = bf16(rope(acc)) on Q/K columns, bf16(acc) on V
  EPI_SWIGLU = 2,      // gate/up interleaved in 32-column blocks: U = silu(g) * u
  EPI_RESID_F32 = 3,   // C = acc + residual, fp32, split row destinations
  EPI_BIAS_BF16 = 4,        // C = bf16(acc + bias)
  EPI_BIAS_RELU_BF16 = 5,   // C = bf16(max(acc + bias, 0))
  EPI_RESID_BIAS_F32 = 6,   // C = residual + (acc + bias), fp32, split row destinations
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
  int rope_cols;       // EPI_QKV_ROPE: columns [0, rope_cols) are rotated
  int hd;              // EPI_QKV_ROPE: head dimension (64 or 128)
  const float* bias;   // EPI_*BIAS*: fp32 [Lw][N], row layer[g] added to every output row
  int q_cols;          // EPI_QKV_ROPE, EPI_BIAS_BF16: columns [0, q_cols) (a multiple of 32)
  float q_scale;       //   are multiplied by q_scale before the bf16 rounding (0 cols: none)
};

// Softmax scale of attention in the base-2 domain, log2(e) / sqrt(hd).  The
// QKV projection folds it into Q for the attention stage of the model, so
// both sides must use this one value.
inline float attention_scale_log2(int hd) { return 1.4426950408889634f / sqrtf((float)hd); }

hipError_t launch_gemm_bf16(int epilogue, const GemmArgs& a, const GroupTable& tab,
                            hipStream_t stream);

// Row-wise RMSNorm of every group's R rows (fp32 in, bf16 out, packed).
hipError_t launch_rmsnorm(int G, int R, int d, int split_in, const GroupTable& tab,
                          const float* gamma, float eps, uint16_t* out, hipStream_t stream);
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
hipError_t launch_gather_tokens(int n, int d, const int32_t* ids, int V, const uint16_t* embed,
                                float* dst, int32_t* bad_flag, hipStream_t stream);
hipError_t launch_copy_rows_bf16(int n, int d, const uint16_t* src, float* dst,
                                 hipStream_t stream);

// Attention over each group's R rows, causal or unmasked; Hq / Hkv must be
// 1, 2 or a multiple of 4.  q_prescaled: Q already carries the softmax scale
// attention_scale_log2(hd) (the QKV epilogue applied it).
hipError_t launch_attention(const uint16_t* qkv, uint16_t* out, int G, int R, int Hq, int Hkv,
                            int hd, bool causal, bool q_prescaled, hipStream_t stream);

// fp32 linear + bias + GELU cell with the split write-back.
hipError_t launch_linear_gelu_f32(int G, int R, int d, int split_in, int split_out,
                                  const GroupTable& tab, const float* W, const float* bias,
                                  hipStream_t stream);

// Weight packing: dst[l][r][k] = src_sel(r)[l][k][col(r)] as bf16.
// interleave == 0: dst row r <- src0 column r (N_dst = N_src).
// interleave == 1: dst row r in block r/64: first 32 rows <- src0 columns,
//                  last 32 rows <- src1 columns (N_dst = 2 N_src).
hipError_t launch_pack(int L, int K, int N_src, const void* src0, const void* src1,
                       int src_is_bf16, int interleave, uint16_t* dst, hipStream_t stream);

}  // namespace rmt
