// Row-wise and layout kernels of the diagonal sweep (gfx950): RMSNorm and
// LayerNorm over every cell of a diagonal, the LLaMA cell's RMSNorm pieces
// that no GEMM epilogue produces (the side outputs of gathered and initial
// rows, and 1/rms per row from the chunk sums), the segment-input gather,
// the fp32 linear+GELU cell, and weight packing.  They are HBM- or
// latency-bound; they read and write full 16-byte (or 8-byte) vectors along
// rows.
#include "kernels.h"

namespace rmt {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// fp32 -> the 16-bit type of a launch: bf16, or fp16 (F16), round to nearest even.
template <bool F16>
__device__ __forceinline__ uint16_t to_16(float f) {
  if constexpr (F16) return __builtin_bit_cast(uint16_t, (_Float16)f);
  else return to_bf16(f);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

enum NormMode : int { NORM_RMS = 0, NORM_LAYER = 1, NORM_CAST = 2 };

// One wave per row, four rows per workgroup.  Row r of group g comes from
// in_lo[g] (r < split_in) or in_hi[g].  The result goes to the packed bf16
// matrix at row g*R + r (unless `out` is null) and, with F32OUT, in fp32 to
// out_lo[g] (r < split_out) or out_hi[g].  Rows of up to 64*4*VPL elements
// stay in registers between the reductions and the scaling, so each input
// byte is read once; wider rows take further passes.  Requires d % 4 == 0.
//   NORM_RMS:   y = x * rsqrt(mean(x^2) + eps) * gamma
//   NORM_LAYER: y = (x - mu) * rsqrt(mean((x - mu)^2) + eps) * gamma + beta
//               (the centred second pass keeps the variance accurate for
//               rows with a large mean)
//   NORM_CAST:  y = x (a bf16 copy of the rows)
// F16: the packed 16-bit result is fp16 instead of bf16.
template <int VPL, int MODE, bool F32OUT, bool F16 = false>
__global__ __launch_bounds__(256) void norm_kernel(int total_rows, int R, int d, int split_in,
                                                   int split_out, GroupTable tab,
                                                   const float* __restrict__ gamma,
                                                   const float* __restrict__ beta, float eps,
                                                   uint16_t* __restrict__ out) {
  constexpr bool LAYER = MODE == NORM_LAYER;
  constexpr bool SCALE = MODE != NORM_CAST;
  const int lane = (int)threadIdx.x & 63;
  const int row = (int)blockIdx.x * 4 + ((int)threadIdx.x >> 6);
  if (row >= total_rows) return;
  const int g = row / R;
  const int r = row - g * R;
  const float* src = r < split_in ? (const float*)tab.in_lo[g] + (size_t)r * d
                                  : (const float*)tab.in_hi[g] + (size_t)(r - split_in) * d;
  const float* gm = SCALE ? gamma + (size_t)tab.layer[g] * d : nullptr;
  const float* bt = LAYER ? beta + (size_t)tab.layer[g] * d : nullptr;
  uint16_t* dst = out ? out + (size_t)row * d : nullptr;
  float* dst32 = nullptr;
  if constexpr (F32OUT)
    dst32 = r < split_out ? (float*)tab.out_lo[g] + (size_t)r * d
                          : (float*)tab.out_hi[g] + (size_t)(r - split_out) * d;
  // LayerNorm's shift is requested with the row too, unless that would take
  // the register count past what keeps several waves per SIMD (wide rows)
  constexpr bool HOIST_BETA = LAYER && VPL <= 8;
  f32x4 v[VPL], w[SCALE ? VPL : 1], bb[HOIST_BETA ? VPL : 1];
  // the row, its gamma (and beta) are requested together, so their latency
  // overlaps the row's instead of following the reductions
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int c = (lane + 64 * j) * 4;
    v[j] = c < d ? *(const f32x4*)(src + c) : f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (SCALE) w[j] = c < d ? *(const f32x4*)(gm + c) : f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (HOIST_BETA) bb[j] = c < d ? *(const f32x4*)(bt + c) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float mu = 0.f, inv = 1.f;
  if constexpr (LAYER) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < VPL; ++j) s += (v[j][0] + v[j][1]) + (v[j][2] + v[j][3]);
    for (int c = (lane + 64 * VPL) * 4; c < d; c += 256) {
      const f32x4 x = *(const f32x4*)(src + c);
      s += (x[0] + x[1]) + (x[2] + x[3]);
    }
    mu = wave_sum(s) / (float)d;
  }
  if constexpr (SCALE) {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int c = (lane + 64 * j) * 4;
      if (!LAYER || c < d) {   // padding lanes hold zeros, which LayerNorm would centre
        const f32x4 x = v[j] - mu;
        ss += x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
      }
    }
    for (int c = (lane + 64 * VPL) * 4; c < d; c += 256) {
      const f32x4 x = *(const f32x4*)(src + c) - mu;
      ss += x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
    }
    ss = wave_sum(ss);
    inv = 1.0f / sqrtf(ss / (float)d + eps);
  }
  auto emit = [&](int c, const f32x4& x, const f32x4& gw, const f32x4& sh) __attribute__((always_inline)) {
    f32x4 y;
    if constexpr (SCALE) {
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = (x[e] - mu) * inv * gw[e];
    } else {
      y = x;
    }
    if constexpr (LAYER) y += sh;
    if (dst) {
      u16x4 o;
      o[0] = to_16<F16>(y[0]);
      o[1] = to_16<F16>(y[1]);
      o[2] = to_16<F16>(y[2]);
      o[3] = to_16<F16>(y[3]);
      *(u16x4*)(dst + c) = o;
    }
    if constexpr (F32OUT) *(f32x4*)(dst32 + c) = y;
  };
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int c = (lane + 64 * j) * 4;
    if (c < d)
      emit(c, v[j], w[SCALE ? j : 0],
           HOIST_BETA ? bb[j] : LAYER ? *(const f32x4*)(bt + c) : zero);
  }
  for (int c = (lane + 64 * VPL) * 4; c < d; c += 256)
    emit(c, *(const f32x4*)(src + c), SCALE ? *(const f32x4*)(gm + c) : zero,
         LAYER ? *(const f32x4*)(bt + c) : zero);
}

// RMSNorm side outputs of four consecutive columns c..c+3 of a row, held by
// one thread of a block that covers the row 1024 columns at a time (thread t
// holds columns 4 t + 1024 j): the 16-bit copy y * gamma, and, from the 16
// threads that share a 64-column chunk, the chunk's sum of squares (a fixed
// butterfly, so every one of the 16 gets the same bits; the chunk's first
// thread stores it).  The 16 threads of a chunk are consecutive lanes of one
// wave, and every lane reaches the exchange (d is a multiple of 64).
// dss points at the row's sum of chunk 0; chunk j's sum is at dss[j * ss_ld].
template <bool F16>
__device__ __forceinline__ void row_side_outputs(const f32x4& y, int c, const float* __restrict__ gamma,
                                                 uint16_t* __restrict__ dst16, float* __restrict__ dss,
                                                 int ss_ld) {
  float ss = (y[0] * y[0] + y[1] * y[1]) + (y[2] * y[2] + y[3] * y[3]);
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) ss += __shfl_xor(ss, o);
  if (c % kChunk == 0) dss[(size_t)(c / kChunk) * ss_ld] = ss;
  const f32x4 g = *(const f32x4*)(gamma + c);
  u16x4 o;
  o[0] = to_16<F16>(y[0] * g[0]);
  o[1] = to_16<F16>(y[1] * g[1]);
  o[2] = to_16<F16>(y[2] * g[2]);
  o[3] = to_16<F16>(y[3] * g[3]);
  *(u16x4*)(dst16 + c) = o;
}

// Embedding lookup of one segment's n token ids into an fp32 slot.  An id
// outside [0, V) reads as a zero row and raises *bad_flag.  With AUX the
// rows' RMSNorm side outputs go to dst16 / dss as well (gain row `gamma`).
template <bool AUX, bool F16>
__global__ __launch_bounds__(256) void gather_tokens_kernel(int d, const int32_t* __restrict__ ids,
                                                            int V, const uint16_t* __restrict__ embed,
                                                            float* __restrict__ dst,
                                                            int32_t* __restrict__ bad_flag,
                                                            const float* __restrict__ gamma,
                                                            uint16_t* __restrict__ dst16,
                                                            float* __restrict__ dss, int ss_ld) {
  const int i = (int)blockIdx.x;
  const int id = ids[i];
  const bool ok = id >= 0 && id < V;
  if (!ok && threadIdx.x == 0) *bad_flag = 1;
  const uint16_t* src = embed + (size_t)(ok ? id : 0) * d;
  float* o = dst + (size_t)i * d;
  for (int c = (int)threadIdx.x * 4; c < d; c += 1024) {
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (ok) {
      const u16x4 h = *(const u16x4*)(src + c);
      v[0] = bf16_to_f32(h[0]);
      v[1] = bf16_to_f32(h[1]);
      v[2] = bf16_to_f32(h[2]);
      v[3] = bf16_to_f32(h[3]);
    }
    *(f32x4*)(o + c) = v;
    if constexpr (AUX)
      row_side_outputs<F16>(v, c, gamma, dst16 + (size_t)i * d, dss + i, ss_ld);
  }
}

// RMSNorm side outputs of fp32 rows that no GEMM epilogue wrote (the initial
// memory M(l, -1)): one block per row; row r uses gain row
// layer0 + (r / rows_per_layer) % L.
template <bool F16>
__global__ __launch_bounds__(256) void norm_aux_rows_kernel(int d, const float* __restrict__ src,
                                                            int rows_per_layer, int L, int layer0,
                                                            const float* __restrict__ gamma,
                                                            uint16_t* __restrict__ dst16,
                                                            float* __restrict__ dss) {
  const int r = (int)blockIdx.x;
  const int q = r / rows_per_layer, i = r - q * rows_per_layer;
  const float* gm = gamma + (size_t)(layer0 + q % L) * d;
  float* ss = dss + (size_t)q * rows_per_layer * (d / kChunk) + i;
  for (int c = (int)threadIdx.x * 4; c < d; c += 1024)
    row_side_outputs<F16>(*(const f32x4*)(src + (size_t)r * d + c), c, gm, dst16 + (size_t)r * d, ss,
                          rows_per_layer);
}

// 1 / sqrt(mean of squares + eps) of every row of every group from its chunk
// sums, added in chunk order (the same formula as norm_kernel's).  Block
// (x, g) covers rows x * 256 .. of group g, so the group's pointers are
// wave-uniform; the chunk sums of a row are fetched 16 at a time (independent
// loads in flight together) and then added in order.
__global__ __launch_bounds__(256) void row_rinv_kernel(int R, int d, int split, NormAux aux, float eps,
                                                       float* __restrict__ rinv) {
  const int g = (int)blockIdx.y;
  const int r = (int)blockIdx.x * 256 + (int)threadIdx.x;
  if (r >= R) return;
  const int nc = d / kChunk;
  const bool lo = r < split;
  const float* ss = lo ? aux.ss_lo[g] + r : aux.ss_hi[g] + (r - split);
  const size_t ld = lo ? (size_t)aux.ss_ld_lo : (size_t)aux.ss_ld_hi;
  constexpr int BATCH = 16;
  float t = 0.f;
  int j = 0;
  for (; j + BATCH <= nc; j += BATCH) {
    float v[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) v[u] = ss[(size_t)(j + u) * ld];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) t += v[u];
  }
  for (; j < nc; ++j) t += ss[(size_t)j * ld];
  rinv[(size_t)g * R + r] = 1.0f / sqrtf(t / (float)d + eps);
}

// bf16 input rows -> fp32 slot (the attention-free cell's segment inputs).
__global__ __launch_bounds__(256) void copy_rows_bf16_kernel(int d, const uint16_t* __restrict__ src,
                                                             float* __restrict__ dst) {
  const size_t base = (size_t)blockIdx.x * d;
  for (int c = (int)threadIdx.x * 4; c < d; c += 1024) {
    const u16x4 h = *(const u16x4*)(src + base + c);
    f32x4 v;
    v[0] = bf16_to_f32(h[0]);
    v[1] = bf16_to_f32(h[1]);
    v[2] = bf16_to_f32(h[2]);
    v[3] = bf16_to_f32(h[3]);
    *(f32x4*)(dst + base + c) = v;
  }
}

// fp32 linear + bias + exact GELU for one diagonal.  Thread (row, col) of
// group g sums A[row][k] W[k][col] for k = 0..d-1 in order with fused
// multiply-adds; rows of A come from in_lo/in_hi, rows of Y go to
// out_lo/out_hi (X(l, s) and M(l, s)).  W is [L][d][d] in the mathematical
// layout, so consecutive threads read consecutive columns.
__global__ __launch_bounds__(256) void linear_gelu_f32_kernel(int R, int d, int split_in, int split_out,
                                                              GroupTable tab, const float* __restrict__ W,
                                                              const float* __restrict__ bias) {
  const int col = (int)blockIdx.x * 64 + ((int)threadIdx.x & 63);
  const int row = (int)blockIdx.y * 4 + ((int)threadIdx.x >> 6);
  const int g = (int)blockIdx.z;
  if (col >= d || row >= R) return;
  const int l = tab.layer[g];
  const float* a = row < split_in ? (const float*)tab.in_lo[g] + (size_t)row * d
                                  : (const float*)tab.in_hi[g] + (size_t)(row - split_in) * d;
  const float* w = W + (size_t)l * d * d + col;
  float acc = 0.f;
  for (int k = 0; k < d; ++k) acc = fmaf(a[k], w[(size_t)k * d], acc);
  const float z = acc + bias[(size_t)l * d + col];
  const float y = 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
  float* o = row < split_out ? (float*)tab.out_lo[g] + (size_t)row * d
                             : (float*)tab.out_hi[g] + (size_t)(row - split_out) * d;
  o[col] = y;
}

// dst[l][r][k] (bf16, or fp16 with DST_F16) from src[l][k][col(r)] through a
// 64 x 64 LDS tile; col(r) per mode (see launch_pack).
template <bool SRC_BF16, bool DST_F16>
__global__ __launch_bounds__(256) void pack_kernel(int K, int N_src, const void* __restrict__ src0,
                                                   const void* __restrict__ src1, int mode, int pair_cols,
                                                   uint16_t* __restrict__ dst) {
  __shared__ uint16_t tile[64][65];
  const int N_dst = mode == PACK_GATE_UP ? 2 * N_src : N_src;
  const int r0 = (int)blockIdx.x * 64;
  const int k0 = (int)blockIdx.y * 64;
  const int l = (int)blockIdx.z;
  const int tx = (int)threadIdx.x & 63;
  const int ty = (int)threadIdx.x >> 6;
  // source column and source tensor of destination row r0 + tx
  const int r = r0 + tx;
  int col = r;
  const void* src = src0;
  if (mode == PACK_GATE_UP) {
    const int blk = r >> 6, j = r & 63;
    col = blk * 32 + (j & 31);
    src = j < 32 ? src0 : src1;
  } else if (mode == PACK_ROPE_PAIRS && r < pair_cols) {
    // 128-wide head h, position p: the 64-column group q = p / 64 holds the
    // head's rotation pairs 32 q .. 32 q + 31, first elements (dimensions
    // 32 q + w) then second elements (64 + 32 q + w)
    const int h = r >> 7, p = r & 127, q = p >> 6, w = p & 63;
    col = h * 128 + (w < 32 ? 32 * q + w : 64 + 32 * q + (w - 32));
  }
  for (int i = ty; i < 64; i += 4) {
    const int k = k0 + i;
    uint16_t v = 0;
    if (k < K && r < N_dst) {
      const size_t idx = ((size_t)l * K + k) * N_src + col;
      if constexpr (DST_F16) {
        const float x = SRC_BF16 ? bf16_to_f32(((const uint16_t*)src)[idx]) : ((const float*)src)[idx];
        v = to_16<true>(x);
      } else {
        if (SRC_BF16) v = ((const uint16_t*)src)[idx];
        else v = to_bf16(((const float*)src)[idx]);
      }
    }
    tile[i][tx] = v;
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int rr = r0 + i;
    const int k = k0 + tx;
    if (rr < N_dst && k < K) dst[((size_t)l * N_dst + rr) * K + k] = tile[tx][i];
  }
}

}  // namespace

template <int MODE, bool F32OUT, bool F16 = false>
hipError_t launch_norm(int G, int R, int d, int split_in, int split_out, const GroupTable& tab,
                       const float* gamma, const float* beta, float eps, uint16_t* out,
                       hipStream_t stream) {
  const int rows = G * R;
  if (rows == 0) return hipSuccess;
  // 8 (16) float4 per lane keep rows of up to 2048 (4096) elements in
  // registers; the smaller variant leaves room for more waves per SIMD
  if (d <= 2048)
    hipLaunchKernelGGL((norm_kernel<8, MODE, F32OUT, F16>), dim3((rows + 3) / 4), dim3(256), 0, stream,
                       rows, R, d, split_in, split_out, tab, gamma, beta, eps, out);
  else
    hipLaunchKernelGGL((norm_kernel<16, MODE, F32OUT, F16>), dim3((rows + 3) / 4), dim3(256), 0, stream,
                       rows, R, d, split_in, split_out, tab, gamma, beta, eps, out);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(int G, int R, int d, int split_in, const GroupTable& tab,
                          const float* gamma, float eps, uint16_t* out, hipStream_t stream, bool f16) {
  if (f16) return launch_norm<NORM_RMS, false, true>(G, R, d, split_in, R, tab, gamma, nullptr, eps, out, stream);
  return launch_norm<NORM_RMS, false>(G, R, d, split_in, R, tab, gamma, nullptr, eps, out, stream);
}

hipError_t launch_layernorm(int G, int R, int d, int split_in, const GroupTable& tab,
                            const float* gamma, const float* beta, float eps, uint16_t* out,
                            hipStream_t stream) {
  return launch_norm<NORM_LAYER, false>(G, R, d, split_in, R, tab, gamma, beta, eps, out, stream);
}

hipError_t launch_layernorm_f32(int G, int R, int d, int split_in, int split_out,
                                const GroupTable& tab, const float* gamma, const float* beta,
                                float eps, uint16_t* out_bf16, hipStream_t stream) {
  return launch_norm<NORM_LAYER, true>(G, R, d, split_in, split_out, tab, gamma, beta, eps, out_bf16,
                                       stream);
}

hipError_t launch_cast_rows(int G, int R, int d, int split_in, const GroupTable& tab, uint16_t* out,
                            hipStream_t stream) {
  return launch_norm<NORM_CAST, false>(G, R, d, split_in, R, tab, nullptr, nullptr, 0.f, out, stream);
}

hipError_t launch_gather_tokens(int n, int d, const int32_t* ids, int V, const uint16_t* embed,
                                float* dst, int32_t* bad_flag, hipStream_t stream, const float* gamma,
                                uint16_t* dst16, float* dss, int ss_ld, bool f16) {
  if (n == 0) return hipSuccess;
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(n), dim3(256), 0, stream, d, ids, V, embed, dst, bad_flag, gamma, dst16, dss,
                       ss_ld);
  };
  if (!dst16) go(gather_tokens_kernel<false, false>);
  else if (d % kChunk != 0 || !gamma || !dss || ss_ld < n) return hipErrorInvalidValue;
  else if (f16) go(gather_tokens_kernel<true, true>);
  else go(gather_tokens_kernel<true, false>);
  return hipGetLastError();
}

hipError_t launch_norm_aux_rows(int rows, int d, const float* src, int rows_per_layer, int L, int layer0,
                                const float* gamma, uint16_t* dst16, float* dss, bool f16,
                                hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  if (d % kChunk != 0 || rows_per_layer < 1 || L < 1) return hipErrorInvalidValue;
  if (f16)
    hipLaunchKernelGGL(norm_aux_rows_kernel<true>, dim3(rows), dim3(256), 0, stream, d, src, rows_per_layer, L,
                       layer0, gamma, dst16, dss);
  else
    hipLaunchKernelGGL(norm_aux_rows_kernel<false>, dim3(rows), dim3(256), 0, stream, d, src, rows_per_layer, L,
                       layer0, gamma, dst16, dss);
  return hipGetLastError();
}

hipError_t launch_row_rinv(int G, int R, int d, int split, const NormAux& aux, float eps, float* rinv,
                           hipStream_t stream) {
  if (G == 0 || R == 0) return hipSuccess;
  if (d % kChunk != 0 || G > kMaxGroups) return hipErrorInvalidValue;
  hipLaunchKernelGGL(row_rinv_kernel, dim3((R + 255) / 256, G), dim3(256), 0, stream, R, d, split, aux, eps, rinv);
  return hipGetLastError();
}

hipError_t launch_copy_rows_bf16(int n, int d, const uint16_t* src, float* dst,
                                 hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_rows_bf16_kernel, dim3(n), dim3(256), 0, stream, d, src, dst);
  return hipGetLastError();
}

hipError_t launch_linear_gelu_f32(int G, int R, int d, int split_in, int split_out,
                                  const GroupTable& tab, const float* W, const float* bias,
                                  hipStream_t stream) {
  if (G == 0) return hipSuccess;
  dim3 grid((d + 63) / 64, (R + 3) / 4, G);
  hipLaunchKernelGGL(linear_gelu_f32_kernel, grid, dim3(256), 0, stream, R, d, split_in,
                     split_out, tab, W, bias);
  return hipGetLastError();
}

hipError_t launch_pack(int L, int K, int N_src, const void* src0, const void* src1,
                       int src_is_bf16, int mode, uint16_t* dst, hipStream_t stream,
                       int dst_f16, int pair_cols) {
  if (mode != PACK_PLAIN && mode != PACK_GATE_UP && mode != PACK_ROPE_PAIRS) return hipErrorInvalidValue;
  if (mode == PACK_ROPE_PAIRS && (pair_cols < 0 || pair_cols % 128 != 0 || pair_cols > N_src))
    return hipErrorInvalidValue;
  const int N_dst = mode == PACK_GATE_UP ? 2 * N_src : N_src;
  dim3 grid((N_dst + 63) / 64, (K + 63) / 64, L);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, K, N_src, src0, src1, mode, pair_cols, dst);
  };
  if (src_is_bf16) {
    if (dst_f16) go(pack_kernel<true, true>);
    else go(pack_kernel<true, false>);
  } else {
    if (dst_f16) go(pack_kernel<false, true>);
    else go(pack_kernel<false, false>);
  }
  return hipGetLastError();
}

}  // namespace rmt
