// Grouped GEMM for one anti-diagonal of the (layer, segment) grid, bf16 MFMA
// with fp32 accumulation, for AMD Instinct MI355X (gfx950).
//
// Every group g is one cell (l, s) of the diagonal: it multiplies its own
// rows A_g (M x K, bf16) by its own layer's weight B_{layer[g]} (stored
// transposed, N x K) -- "GroupedGEMM Operations" and "GPU Kernel
// Optimization" in the Architecture Overview of the skill page "Diagonal
// Batching for Recurrent Memory Transformers": one launch covers all cells of
// a diagonal, whatever their number.
//
// Tiling: a workgroup of 4 wave64s computes a 128 x 256 tile; each wave a
// 64 x 128 sub-tile as 2 x 4 blocks of v_mfma_f32_32x32x16_bf16.  128 divides
// the cell height R = n + m of the 1B/8B workloads (1152, 2176), so no tile
// straddles two groups.  K is consumed 64 at a time through LDS (row stride
// 72 elements: 144 bytes keeps 16-byte reads of 32 consecutive rows free of
// bank conflicts); the next K slice is fetched into registers while the
// current one feeds the MFMAs.  Every output element is produced by one
// thread with the same K order whatever G is, so a cell's result does not
// depend on which diagonal (or the sequential sweep) it runs in.
#include "kernels.h"

namespace rmt {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128;
constexpr int BN = 256;
constexpr int BK = 64;
constexpr int LDK = BK + 8;
constexpr int NT = 256;

__device__ __forceinline__ uint16_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Workgroups are handed to the 8 XCDs round-robin (id mod 8).  Renumber them
// so that each XCD receives one contiguous run of tiles: tiles that share a
// weight panel then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int nb) {
  const int per = nb >> 3, rem = nb & 7;
  const int xcd = bid & 7, idx = bid >> 3;
  return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

template <int EPI>
__global__ __launch_bounds__(NT, 2) void gemm_bf16_kernel(GemmArgs a, GroupTable tab) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[BM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[BN * LDK];

  const int tiles_m = (a.M + BM - 1) / BM;
  const int tiles_n = (a.N + BN - 1) / BN;
  const int per_group = tiles_m * tiles_n;
  const int bid = xcd_remap((int)blockIdx.x, (int)gridDim.x);
  const int g = bid / per_group;
  const int rem = bid - g * per_group;
  const int tn = rem / tiles_m;        // m fastest: consecutive tiles share B
  const int tm = rem - tn * tiles_m;
  const int tid = (int)threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;
  const int wn = wave & 1;

  const int K = a.K;
  const uint16_t* Ag = a.A + ((size_t)g * a.M + (size_t)tm * BM) * K;
  const uint16_t* Bg = a.B + ((size_t)tab.layer[g] * a.N + (size_t)tn * BN) * K;
  const int m_valid = min(BM, a.M - tm * BM);
  const int n_valid = min(BN, a.N - tn * BN);

  const int lrow = tid >> 3;
  const int lk = (tid & 7) * 8;
  u32x4 ra[BM / 32];
  u32x4 rb[BN / 32];
  const u32x4 zero = {0u, 0u, 0u, 0u};

  auto load = [&](int k0) {
    const bool kin = (k0 + lk) < K;
#pragma unroll
    for (int i = 0; i < BM / 32; ++i) {
      const int r = lrow + 32 * i;
      ra[i] = (kin && r < m_valid) ? *(const u32x4*)(Ag + (size_t)r * K + k0 + lk) : zero;
    }
#pragma unroll
    for (int i = 0; i < BN / 32; ++i) {
      const int r = lrow + 32 * i;
      rb[i] = (kin && r < n_valid) ? *(const u32x4*)(Bg + (size_t)r * K + k0 + lk) : zero;
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < BM / 32; ++i) *(u32x4*)(sA + (lrow + 32 * i) * LDK + lk) = ra[i];
#pragma unroll
    for (int i = 0; i < BN / 32; ++i) *(u32x4*)(sB + (lrow + 32 * i) * LDK + lk) = rb[i];
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][t][e] = 0.f;

  // Lane l feeds row (l % 32) of its A/B blocks with 8 consecutive k values.
  // Within one 64-wide K slice, lanes 0-31 cover k 0..31 and lanes 32-63 cover
  // k 32..63 over the four MFMA steps; A and B use the same assignment, so
  // each MFMA still sums matching k.
  const int r32 = lane & 31;
  const int kofs = (lane >> 5) * 32;
  const int nk = (K + BK - 1) / BK;
  load(0);
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();
    store();
    __syncthreads();
    if (kt + 1 < nk) load((kt + 1) * BK);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x8 af[2], bfr[4];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = __builtin_bit_cast(bf16x8, *(const u32x4*)(sA + (wm * 64 + i * 32 + r32) * LDK + kofs + 8 * j));
#pragma unroll
      for (int t = 0; t < 4; ++t)
        bfr[t] = __builtin_bit_cast(bf16x8, *(const u32x4*)(sB + (wn * 128 + t * 32 + r32) * LDK + kofs + 8 * j));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int t = 0; t < 4; ++t)
          acc[i][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[t], acc[i][t], 0, 0, 0);
    }
  }

  // Accumulator layout of a 32x32 block: element e of lane l sits at
  // row 8*(e/4) + 4*(l/32) + e%4, column l%32.
  const int row_base = tm * BM + wm * 64 + 4 * (lane >> 5);
  const int col_base = tn * BN + wn * 128 + r32;

  if constexpr (EPI == EPI_STORE_BF16) {
    uint16_t* C = (uint16_t*)tab.out_lo[g];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = row_base + i * 32 + 8 * (e >> 2) + (e & 3);
        if (row >= a.M) continue;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int col = col_base + t * 32;
          if (col < a.N) C[(size_t)row * a.ld_out + col] = to_bf16(acc[i][t][e]);
        }
      }
  } else if constexpr (EPI == EPI_QKV_ROPE) {
    // The wave's 128 columns start on a head boundary (128 is a multiple of
    // hd), so column c < hd/2 of a head and its partner c + hd/2 sit in the
    // same lane, in blocks t and t + hd/64.
    uint16_t* C = (uint16_t*)tab.out_lo[g];
    const int P = a.hd >> 6;
    const int half = a.hd >> 1;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (((t / P) & 1) != 0) continue;
      const int col = col_base + t * 32;
      if (col >= a.N) continue;
      const bool rot = col < a.rope_cols;
      const int hc = col % a.hd;
      const int tp = t + P;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = row_base + i * 32 + 8 * (e >> 2) + (e & 3);
          if (row >= a.M) continue;
          float x1 = acc[i][t][e];
          float x2 = 0.f;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (q == tp) x2 = acc[i][q][e];
          float y1 = x1, y2 = x2;
          if (rot) {
            const float2 cs = a.rope[(size_t)row * half + hc];
            y1 = x1 * cs.x - x2 * cs.y;
            y2 = x2 * cs.x + x1 * cs.y;
          }
          C[(size_t)row * a.ld_out + col] = to_bf16(y1);
          C[(size_t)row * a.ld_out + col + half] = to_bf16(y2);
        }
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    // Packed columns come in 64-wide blocks: 32 gate columns then the 32 up
    // columns of the same outputs; output column = block * 32 + (l % 32).
    uint16_t* U = (uint16_t*)tab.out_lo[g];
#pragma unroll
    for (int t = 0; t < 4; t += 2) {
      const int col = col_base + t * 32;
      if (col >= a.N) continue;
      const int ocol = (col >> 6) * 32 + r32;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = row_base + i * 32 + 8 * (e >> 2) + (e & 3);
          if (row >= a.M) continue;
          const float gt = acc[i][t][e];
          const float up = acc[i][t + 1][e];
          const float u = gt / (1.0f + expf(-gt)) * up;
          U[(size_t)row * a.ld_out + ocol] = to_bf16(u);
        }
    }
  } else {  // EPI_RESID_F32
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = row_base + i * 32 + 8 * (e >> 2) + (e & 3);
        if (row >= a.M) continue;
        const float* res = row < a.split_in
                               ? (const float*)tab.in_lo[g] + (size_t)row * a.ld_res
                               : (const float*)tab.in_hi[g] + (size_t)(row - a.split_in) * a.ld_res;
        float* out = row < a.split_out
                         ? (float*)tab.out_lo[g] + (size_t)row * a.ld_out
                         : (float*)tab.out_hi[g] + (size_t)(row - a.split_out) * a.ld_out;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int col = col_base + t * 32;
          if (col < a.N) out[col] = acc[i][t][e] + res[col];
        }
      }
  }
}

}  // namespace

hipError_t launch_gemm_bf16(int epilogue, const GemmArgs& a, const GroupTable& tab,
                            hipStream_t stream) {
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN) * tab.G;
  if (tiles == 0) return hipSuccess;
  dim3 grid(tiles), block(NT);
  switch (epilogue) {
    case EPI_STORE_BF16:
      hipLaunchKernelGGL(gemm_bf16_kernel<EPI_STORE_BF16>, grid, block, 0, stream, a, tab);
      break;
    case EPI_QKV_ROPE:
      hipLaunchKernelGGL(gemm_bf16_kernel<EPI_QKV_ROPE>, grid, block, 0, stream, a, tab);
      break;
    case EPI_SWIGLU:
      hipLaunchKernelGGL(gemm_bf16_kernel<EPI_SWIGLU>, grid, block, 0, stream, a, tab);
      break;
    case EPI_RESID_F32:
      hipLaunchKernelGGL(gemm_bf16_kernel<EPI_RESID_F32>, grid, block, 0, stream, a, tab);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rmt
