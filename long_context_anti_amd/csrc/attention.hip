// Causal grouped-query attention inside each cell of a diagonal (gfx950).
//
// A cell (l, s) attends over its own R = m + n rows [memory; segment] with a
// lower-triangular mask; query head h reads KV head h / (Hq / Hkv).  All
// cells of a diagonal are covered by one launch (grid z = cell).
//
// One workgroup = 4 wave64s = 4 query heads that share one KV head, over a
// block of QB query rows.  K and V come through LDS 64 keys at a time and are
// shared by the 4 heads.  The kernel works on transposed scores
// S^T = K Q^T (v_mfma_f32_16x16x32_bf16): the accumulator layout of S^T then
// matches the B-operand layout that O^T += V^T P^T needs, so the
// probabilities go from the softmax straight into the second MFMA without a
// trip through LDS.  Online softmax in fp32 with exp2.
#include "kernels.h"

namespace rmt {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int KB = 64;  // keys per LDS block

__device__ __forceinline__ uint16_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return (uint32_t)to_bf16(lo) | ((uint32_t)to_bf16(hi) << 16);
}

template <int HD, int QB>
__global__ __launch_bounds__(256, 2) void attention_kernel(const uint16_t* __restrict__ qkv,
                                                           uint16_t* __restrict__ out, int R,
                                                           int Hq, int Hkv, float scale_log2) {
  constexpr int QT = QB / 16;   // query tiles of 16 per wave
  constexpr int KS = HD / 32;   // k-steps of 32 over the head dimension
  constexpr int HT = HD / 16;   // head-dimension tiles of 16 in O^T
  constexpr int LDK = HD + 8;   // sK row stride (elements)
  constexpr int LDV = KB + 8;   // sVt row stride (elements)
  __shared__ __attribute__((aligned(16))) uint16_t sK[KB * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[HD * LDV];

  const int tid = (int)threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c16 = lane & 15;     // column within a 16-wide tile
  const int g4 = lane >> 4;      // lane group 0..3

  const int nqb = (R + QB - 1) / QB;
  const int q0 = (nqb - 1 - (int)blockIdx.x) * QB;   // longest blocks first
  const int rep = Hq / Hkv;
  const int quads = rep >> 2;
  const int kvh = (int)blockIdx.y / quads;
  const int h = kvh * rep + ((int)blockIdx.y % quads) * 4 + wave;
  const int g = (int)blockIdx.z;
  const int ld = (Hq + 2 * Hkv) * HD;
  const uint16_t* base = qkv + (size_t)g * R * ld;
  const uint16_t* Kp = base + (size_t)(Hq + kvh) * HD;
  const uint16_t* Vp = base + (size_t)(Hq + Hkv + kvh) * HD;

  // Q^T as the B operand: lane holds Q[q0 + 16 qt + c16][32 ks + 8 g4 + 0..7].
  bf16x8 qf[QT][KS];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int q = q0 + 16 * qt + c16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (q < R) v = *(const u32x4*)(base + (size_t)q * ld + (size_t)h * HD + 32 * ks + 8 * g4);
      qf[qt][ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x4 o[HT][QT];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) o[ht][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrow[QT], lrow[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    mrow[qt] = -INFINITY;
    lrow[qt] = 0.f;
  }

  const int kend = min(q0 + QB, R);          // keys needed: [0, kend)
  const int nkb = (kend + KB - 1) / KB;
  constexpr int CH = HD / 8;                  // 16-byte chunks per key row
  for (int kb = 0; kb < nkb; ++kb) {
    const int k0 = kb * KB;
    __syncthreads();
    for (int c = tid; c < KB * CH; c += 256) {
      const int r = c / CH;
      const int cc = (c % CH) * 8;
      u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (k0 + r < R) {
        kv = *(const u32x4*)(Kp + (size_t)(k0 + r) * ld + cc);
        vv = *(const u32x4*)(Vp + (size_t)(k0 + r) * ld + cc);
      }
      *(u32x4*)(sK + r * LDK + cc) = kv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sVt[(cc + 2 * e) * LDV + r] = (uint16_t)(vv[e] & 0xffffu);
        sVt[(cc + 2 * e + 1) * LDV + r] = (uint16_t)(vv[e] >> 16);
      }
    }
    __syncthreads();

    // S^T block: 64 keys x QB queries.  Lane holds keys 16 kt + 4 g4 + j of
    // query column 16 qt + c16.
    f32x4 s[4][QT];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) s[kt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const bf16x8 kf = __builtin_bit_cast(
            bf16x8, *(const u32x4*)(sK + (16 * kt + c16) * LDK + 32 * ks + 8 * g4));
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          s[kt][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[qt][ks], s[kt][qt], 0, 0, 0);
      }

    const bool need_mask = (k0 + KB - 1 > q0) || (k0 + KB > R);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const int q = q0 + 16 * qt + c16;
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float v = s[kt][qt][j] * scale_log2;
          if (need_mask) {
            const int key = k0 + 16 * kt + 4 * g4 + j;
            if (key > q || key >= R) v = -INFINITY;
          }
          s[kt][qt][j] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(mrow[qt], mx);
      const float corr = exp2f(mrow[qt] - mnew);
      float sum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p = exp2f(s[kt][qt][j] - mnew);
          s[kt][qt][j] = p;
          sum += p;
        }
      sum += __shfl_xor(sum, 16);
      sum += __shfl_xor(sum, 32);
      lrow[qt] = lrow[qt] * corr + sum;
      mrow[qt] = mnew;
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) o[ht][qt] *= corr;
    }

    // O^T += V^T P^T over two 32-key steps.  In step ks2 lane slot e < 4 is key
    // 32 ks2 + 4 g4 + e and slot e >= 4 is key 32 ks2 + 16 + 4 g4 + (e - 4),
    // matching where the S^T accumulator left those probabilities.
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      bf16x8 pf[QT];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        u32x4 w;
        w[0] = pack2(s[2 * ks2][qt][0], s[2 * ks2][qt][1]);
        w[1] = pack2(s[2 * ks2][qt][2], s[2 * ks2][qt][3]);
        w[2] = pack2(s[2 * ks2 + 1][qt][0], s[2 * ks2 + 1][qt][1]);
        w[3] = pack2(s[2 * ks2 + 1][qt][2], s[2 * ks2 + 1][qt][3]);
        pf[qt] = __builtin_bit_cast(bf16x8, w);
      }
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        const uint16_t* vrow = sVt + (16 * ht + c16) * LDV + 32 * ks2 + 4 * g4;
        u32x4 w;
        const u32x2 lo = *(const u32x2*)(vrow);
        const u32x2 hi = *(const u32x2*)(vrow + 16);
        w[0] = lo[0];
        w[1] = lo[1];
        w[2] = hi[0];
        w[3] = hi[1];
        const bf16x8 vf = __builtin_bit_cast(bf16x8, w);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          o[ht][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[qt], o[ht][qt], 0, 0, 0);
      }
    }
  }

  // O^T accumulator: lane holds head dims 16 ht + 4 g4 + j of query 16 qt + c16.
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int q = q0 + 16 * qt + c16;
    if (q >= R) continue;
    const float inv = 1.0f / lrow[qt];
    uint16_t* orow = out + ((size_t)g * R + q) * (size_t)(Hq * HD) + (size_t)h * HD;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      u32x2 w;
      w[0] = pack2(o[ht][qt][0] * inv, o[ht][qt][1] * inv);
      w[1] = pack2(o[ht][qt][2] * inv, o[ht][qt][3] * inv);
      *(u32x2*)(orow + 16 * ht + 4 * g4) = w;
    }
  }
}

}  // namespace

hipError_t launch_attention(const uint16_t* qkv, uint16_t* out, int G, int R, int Hq, int Hkv,
                            int hd, hipStream_t stream) {
  if (G == 0 || R == 0) return hipSuccess;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)hd);
  const int quads = (Hq / Hkv) / 4;
  if (hd == 64) {
    constexpr int QB = 64;
    dim3 grid((R + QB - 1) / QB, Hkv * quads, G);
    hipLaunchKernelGGL((attention_kernel<64, QB>), grid, dim3(256), 0, stream, qkv, out, R, Hq,
                       Hkv, scale_log2);
  } else if (hd == 128) {
    constexpr int QB = 32;
    dim3 grid((R + QB - 1) / QB, Hkv * quads, G);
    hipLaunchKernelGGL((attention_kernel<128, QB>), grid, dim3(256), 0, stream, qkv, out, R, Hq,
                       Hkv, scale_log2);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rmt
