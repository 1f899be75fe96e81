// Attention inside each cell of a diagonal (gfx950): a cell (l, s) attends
// over its own R = m + n rows [memory; segment], either causally (lower-
// triangular mask: the LLaMA-shaped cell) or with every row seeing every row
// (the encoder-layer cell); query head h reads KV head h / (Hq / Hkv).  All
// cells of a diagonal are covered by one launch (grid z = cell).
//
// One workgroup = 4 wave64s that share one KV head: 4 of its query heads over
// one block of QB query rows when Hq / Hkv is a multiple of 4, 2 heads x 2
// query blocks when it is 2, one head x 4 query blocks when it is 1 (plain
// multi-head attention).  K and V blocks of 64 keys go through a two-slot LDS
// ring (the next block is fetched into registers while the current one is
// used) and are shared by the 4 waves.
//
// Per 64-key block each wave computes transposed scores S^T = K Q^T with
// v_mfma_f32_16x16x32_bf16: the S^T accumulator layout is exactly the
// B-operand layout that O^T += V^T P^T needs, so probabilities go from the
// softmax straight into the second MFMA.  V^T operands come from row-major V
// through the transposing LDS read ds_read_b64_tr_b16.  The softmax is
// online in fp32 and base 2 (one FMA + one v_exp_f32 per score); the running
// output is rescaled only when a row maximum grows by more than 2^8, which
// keeps every probability below 256 and leaves O / l unchanged.  At
// head_dim 64 a key block costs a wave more VALU cycles than MFMA cycles
// (v_exp_f32 issues at a quarter of the FMA rate), so VALU work is kept
// off the per-block path where it can be: the row sums l come from one more
// MFMA per step against a row of ones -- the sum of exactly the bf16
// probabilities that multiply V -- and the row maxima cross lane groups
// (v_permlane16/32_swap) only when a rescale is due.
#include "kernels.h"

namespace rmt {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int KB = 64;            // keys per block
constexpr float RESCALE_LOG2 = 8.0f;

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;              // v_cvt_pk_bf16_f32: round to nearest even
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Maximum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lane groups
// that hold one query column), with the gfx950 cross-row lane swaps.
__device__ __forceinline__ float max_over_groups(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Workgroups are handed to the 8 XCDs round-robin (id mod 8); this
// renumbering gives each XCD one contiguous run of ids.
__device__ __forceinline__ int xcd_remap(int bid, int nb) {
  const int per = nb >> 3, rem = nb & 7;
  const int xcd = bid & 7, idx = bid >> 3;
  return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

template <int HD, int QB, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void attention_kernel(const uint16_t* __restrict__ qkv,
                                                           uint16_t* __restrict__ out, int R,
                                                           int Hq, int Hkv, float scale_log2) {
  constexpr int QT = QB / 16;     // query tiles of 16 per wave
  constexpr int KS = HD / 32;     // k-steps of 32 over the head dimension
  constexpr int HT = HD / 16;     // head-dimension tiles of 16 in O^T
  constexpr int LDK = HD + 8;     // K row stride: 16-byte reads of 16 rows hit distinct banks
  constexpr int LDV = HD + 16;    // V row stride: 8-byte transposing reads of 8 rows tile the banks
  constexpr int CH = HD / 8;      // 16-byte chunks per key row
  constexpr int LOADS = KB * CH / 256;   // chunks per thread per block, for K and for V
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][KB * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][KB * LDV];

  const int tid = (int)threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c16 = lane & 15;      // column within a 16-wide tile
  const int g4 = lane >> 4;       // lane group 0..3

  // The workgroup's waves: hw query heads of one KV head x qw query blocks.
  const int rep = Hq / Hkv;
  const int hw = rep >= 4 ? 4 : rep;
  const int qw = 4 / hw;
  const int hgroups = rep / hw;                 // workgroups per KV head along y
  // Workgroups go to the 8 XCDs round-robin; renumber them so that each XCD
  // receives a contiguous run of (cell, KV head) groups and the K/V rows of a
  // group are fetched into one L2 only.  Within a group the query blocks keep
  // their order, longest first.
  const int nqb = (R + QB - 1) / QB;
  const int nqg = (nqb + qw - 1) / qw;          // groups of qw query blocks (grid x)
  const int ny = (int)gridDim.y;
  const int lin = xcd_remap((int)(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z)),
                            (int)(gridDim.x * gridDim.y * gridDim.z));
  const int bx = lin % nqg;
  const int by = (lin / nqg) % ny;
  const int qg0 = (nqg - 1 - bx) * qw * QB;    // the workgroup's first query row
  const int q0 = qg0 + (wave / hw) * QB;        // this wave's query block (may start at or past R)
  const int kvh = by / hgroups;
  const int h = kvh * rep + (by % hgroups) * hw + wave % hw;
  const int g = lin / (nqg * ny);
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
  // mref: reference maximum in the scaled (log2) domain.  osum: row sums of
  // the bf16 probabilities, from one more MFMA per step whose A operand has a
  // row of ones (row 0, i.e. lanes c16 == 0): element 0 of lane c16 < 16
  // holds the sum for query 16 qt + c16, and the rescaling treats it like O.
  float mref[QT];
  f32x4 osum[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    mref[qt] = -INFINITY;
    osum[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const uint32_t one2 = c16 == 0 ? 0x3F803F80u : 0u;   // two bf16 ones, or zeros
  const bf16x8 ones_row = __builtin_bit_cast(bf16x8, u32x4{one2, one2, one2, one2});

  // K/V block loads: thread chunk c -> key c / CH, columns (c % CH) * 8.
  u32x4 rk[LOADS], rv[LOADS];
  auto fetch = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int c = tid + 256 * i;
      const int r = c / CH;
      const int cc = (c % CH) * 8;
      rk[i] = u32x4{0u, 0u, 0u, 0u};
      rv[i] = u32x4{0u, 0u, 0u, 0u};
      if (k0 + r < R) {
        rk[i] = *(const u32x4*)(Kp + (size_t)(k0 + r) * ld + cc);
        rv[i] = *(const u32x4*)(Vp + (size_t)(k0 + r) * ld + cc);
      }
    }
  };
  auto stash = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int c = tid + 256 * i;
      const int r = c / CH;
      const int cc = (c % CH) * 8;
      *(u32x4*)(&sK[slot][r * LDK + cc]) = rk[i];
      *(u32x2*)(&sV[slot][r * LDV + cc]) = u32x2{rv[i][0], rv[i][1]};
      *(u32x2*)(&sV[slot][r * LDV + cc + 4]) = u32x2{rv[i][2], rv[i][3]};
    }
  };

  // keys needed by any of the workgroup's query rows: [0, kend)
  const int kend = CAUSAL ? min(qg0 + qw * QB, R) : R;
  const int nkb = (kend + KB - 1) / KB;
  fetch(0);
  stash(0);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int slot = kb & 1;
    const int k0 = kb * KB;
    if (kb + 1 < nkb) fetch(k0 + KB);
    const uint16_t* K_ = sK[slot];
    const uint16_t* V_ = sV[slot];

    // S^T block: 64 keys x QB queries.  Lane holds keys 16 kt + 4 g4 + j of
    // query column 16 qt + c16 (raw, unscaled scores).
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
            bf16x8, *(const u32x4*)(K_ + (16 * kt + c16) * LDK + 32 * ks + 8 * g4));
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          s[kt][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[qt][ks], s[kt][qt], 0, 0, 0);
      }

    // Masked scores: keys past the cell's end and, when causal, keys after
    // the query.  (A causal block wholly after this wave's rows masks them
    // all: its probabilities are exactly zero.)
    if ((CAUSAL && k0 + KB - 1 > q0) || (k0 + KB > R)) {   // wave-uniform
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const int q = q0 + 16 * qt + c16;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int key = k0 + 16 * kt + 4 * g4 + j;
            if ((CAUSAL && key > q) || key >= R) s[kt][qt][j] = -INFINITY;
          }
      }
    }

    // Lane-local maxima decide whether to rescale: a query's maximum over its
    // four lane groups crosses the threshold exactly when one lane's does, so
    // the cross-group maximum is needed only inside the (rare) rescale.
    bool need_rescale = false;
    float mloc[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {   // three-input maxima (v_max3_f32)
        mx = fmaxf(fmaxf(mx, s[kt][qt][0]), s[kt][qt][1]);
        mx = fmaxf(fmaxf(mx, s[kt][qt][2]), s[kt][qt][3]);
      }
      mloc[qt] = mx;
      need_rescale |= mx * scale_log2 > mref[qt] + RESCALE_LOG2;
    }
    if (__any(need_rescale)) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const float m2 = fmaxf(mref[qt], max_over_groups(mloc[qt]) * scale_log2);
        const float corr = __builtin_amdgcn_exp2f(mref[qt] - m2);   // 0 on the first block
        mref[qt] = m2;
        osum[qt] *= corr;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) o[ht][qt] *= corr;
      }
    }
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          s[kt][qt][j] = __builtin_amdgcn_exp2f(fmaf(s[kt][qt][j], scale_log2, -mref[qt]));

    // O^T += V^T P^T over two 32-key steps.  In step ks2, operand slot e < 4
    // is key 32 ks2 + 4 g4 + e and slot e >= 4 is key 32 ks2 + 16 + 4 g4 +
    // (e - 4), matching where the S^T accumulator left those probabilities.
    // The transposing read: lane j of each 16-lane group points at row
    // key0 + j / 4, columns 4 (j % 4) .. +3; lane i receives column i of the
    // four rows.
    const int tr_row = 4 * g4 + (c16 >> 2);
    const int tr_col = 4 * (c16 & 3);
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      bf16x8 pf[QT];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        u32x4 w;
        w[0] = pack_bf16(s[2 * ks2][qt][0], s[2 * ks2][qt][1]);
        w[1] = pack_bf16(s[2 * ks2][qt][2], s[2 * ks2][qt][3]);
        w[2] = pack_bf16(s[2 * ks2 + 1][qt][0], s[2 * ks2 + 1][qt][1]);
        w[3] = pack_bf16(s[2 * ks2 + 1][qt][2], s[2 * ks2 + 1][qt][3]);
        pf[qt] = __builtin_bit_cast(bf16x8, w);
        osum[qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones_row, pf[qt], osum[qt], 0, 0, 0);
      }
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        const uint16_t* v0 = V_ + (32 * ks2 + tr_row) * LDV + 16 * ht + tr_col;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(v0));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(v0 + 16 * LDV));
        u32x4 w;
        const u32x2 wl = __builtin_bit_cast(u32x2, lo);
        const u32x2 wh = __builtin_bit_cast(u32x2, hi);
        w[0] = wl[0];
        w[1] = wl[1];
        w[2] = wh[0];
        w[3] = wh[1];
        const bf16x8 vf = __builtin_bit_cast(bf16x8, w);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          o[ht][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[qt], o[ht][qt], 0, 0, 0);
      }
    }

    if (kb + 1 < nkb) stash(slot ^ 1);
    __syncthreads();
  }

  // O^T accumulator: lane holds head dims 16 ht + 4 g4 + j of query 16 qt + c16.
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int q = q0 + 16 * qt + c16;
    const float lsum = __shfl(osum[qt][0], c16);   // from lane c16 (lane group 0)
    if (q >= R) continue;
    const float inv = 1.0f / lsum;
    uint16_t* orow = out + ((size_t)g * R + q) * (size_t)(Hq * HD) + (size_t)h * HD;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      u32x2 w;
      w[0] = pack_bf16(o[ht][qt][0] * inv, o[ht][qt][1] * inv);
      w[1] = pack_bf16(o[ht][qt][2] * inv, o[ht][qt][3] * inv);
      *(u32x2*)(orow + 16 * ht + 4 * g4) = w;
    }
  }
}

}  // namespace

hipError_t launch_attention(const uint16_t* qkv, uint16_t* out, int G, int R, int Hq, int Hkv,
                            int hd, bool causal, hipStream_t stream) {
  if (G == 0 || R == 0) return hipSuccess;
  const int rep = Hq / Hkv;
  if (Hkv < 1 || Hq % Hkv != 0 || !(rep == 1 || rep == 2 || rep % 4 == 0)) return hipErrorInvalidValue;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)hd);
  constexpr int QB = 32;   // measured faster than 64: lower register use, more waves
  const int hw = rep >= 4 ? 4 : rep;
  const int qw = 4 / hw;
  const int nqb = (R + QB - 1) / QB;
  const dim3 grid((nqb + qw - 1) / qw, Hkv * (rep / hw), G);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, qkv, out, R, Hq, Hkv, scale_log2);
  };
  if (hd == 64) {
    if (causal) go(attention_kernel<64, QB, true>);
    else go(attention_kernel<64, QB, false>);
  } else if (hd == 128) {
    if (causal) go(attention_kernel<128, QB, true>);
    else go(attention_kernel<128, QB, false>);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rmt
