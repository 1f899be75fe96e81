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
// ring shared by the 4 waves: buffer loads write the next block straight into
// LDS (no staging registers) while the current one is used.  LDS rows are
// unpadded; their 16-byte chunks are XOR-swizzled per row so that both the
// K reads and the transposing V reads are free of bank conflicts.
//
// Per 64-key block each wave computes transposed scores S^T = K Q^T with
// v_mfma_f32_16x16x32_bf16: the S^T accumulator layout is exactly the
// B-operand layout that O^T += V^T P^T needs, so probabilities go from the
// softmax straight into the second MFMA.  V^T operands come from row-major V
// through the transposing LDS read ds_read_b64_tr_b16.  The softmax is
// online in fp32 and base 2.  In the model, Q arrives multiplied by
// log2(e) / sqrt(hd) (the QKV epilogue applies it before the bf16 rounding)
// and each score MFMA starts from minus the row's reference maximum, so its
// result is the exponent itself: one v_exp_f32 per score and nothing else.
// (That sum of -m and the products is rounded at the scale of max(|m|, the
// products), which stays far below the bf16 rounding of the probabilities
// for any realistic score range.)  Called on its own, with unscaled Q, the
// kernel spends one FMA per score instead.  The running output is rescaled
// only when a row maximum grows by more than 2^8, which keeps every
// probability below 256 and leaves O / l unchanged.  At
// head_dim 64 a key block costs a wave more VALU cycles than MFMA cycles
// (v_exp_f32 issues at about a third of the FMA rate, measured), so VALU work is kept
// off the per-block path where it can be: the row sums l come from one more
// MFMA per step against a row of ones -- the sum of exactly the bf16
// probabilities that multiply V -- and the row maxima cross lane groups
// (v_permlane16/32_swap) only when a rescale is due.
#include "kernels.h"

namespace rmt {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int KB = 64;            // keys per block
constexpr float RESCALE_LOG2 = 8.0f;
constexpr int BUF_FLAGS = 0x00020000;        // raw buffer, 32-bit data format

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// The 16-bit type of Q/K/V, the probabilities and the output: bf16, or IEEE
// half (F16).  `pack` rounds two fp32 values to nearest even
// (v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32); `one2` is a packed pair of ones.
template <bool F16>
struct Half16 {
  typedef __bf16 x8 __attribute__((ext_vector_type(8)));
  typedef __bf16 x2 __attribute__((ext_vector_type(2)));
  static constexpr uint32_t one2 = 0x3F803F80u;
  static __device__ __forceinline__ f32x4 mfma(x8 a, x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    x2 v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
  }
};
template <>
struct Half16<true> {
  typedef _Float16 x8 __attribute__((ext_vector_type(8)));
  typedef _Float16 x2 __attribute__((ext_vector_type(2)));
  static constexpr uint32_t one2 = 0x3C003C00u;
  static __device__ __forceinline__ f32x4 mfma(x8 a, x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    x2 v;
    v[0] = (_Float16)lo;
    v[1] = (_Float16)hi;
    return __builtin_bit_cast(uint32_t, v);
  }
};

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

// Chunk permutation of LDS row r, the same for K and V: logical 16-byte chunk
// c sits at physical chunk c ^ swz(r), which depends on r mod 16 only (an XOR
// maps chunk pairs to pairs, as the V reads need).  K is read 16 bytes per
// lane from 16 consecutive rows at one logical chunk; V through 8-byte
// transposing reads that take 32 bytes (a chunk pair) from each of 4
// consecutive rows per 16 lanes.  Chosen by measurement on gfx950 (bank-
// conflict counter and timing of both read patterns, every candidate): these
// keep both patterns conflict free, at 4 LDS cycles per 16-byte wave read and
// 2 per transposing one.  A permutation that a plain 64-bank model clears,
// which earlier versions used, made the K reads 2-way conflicted.
template <int HD>
__device__ __forceinline__ int swz(int r) {
  if constexpr (HD == 64) return r & 6;
  else return 2 * (r & 7);
}

// One wave-wide 16-byte-per-lane buffer load into LDS: lane L's bytes land
// at dst + 16 L.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rs, uint8_t* dst, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)dst, 16, voff, soff, 0, 0);
}

template <int HD, int QB, bool CAUSAL, bool QPRE, bool F16>
__global__ __launch_bounds__(256, HD == 64 ? 4 : 2) void attention_kernel(const uint16_t* __restrict__ qkv,
                                                           uint16_t* __restrict__ out, int R,
                                                           int Hq, int Hkv, float scale_log2) {
  using H = Half16<F16>;
  typedef typename H::x8 op8;
  constexpr int QT = QB / 16;     // query tiles of 16 per wave
  constexpr int KS = HD / 32;     // k-steps of 32 over the head dimension
  constexpr int HT = HD / 16;     // head-dimension tiles of 16 in O^T
  constexpr int ROWB = HD * 2;    // bytes per K / V row in LDS (unpadded)
  constexpr int CPR = HD / 8;     // 16-byte chunks per row
  constexpr int RPL = 64 / CPR;   // rows per wave-wide 1 KiB load
  constexpr int PPW = KB / RPL / 4;   // such loads per wave per block, for K and for V
  static_assert(KB * ROWB == 4 * PPW * 1024, "a block is whole 1 KiB loads, dealt evenly");
  __shared__ __attribute__((aligned(1024))) uint8_t sK[2][KB * ROWB];
  __shared__ __attribute__((aligned(1024))) uint8_t sV[2][KB * ROWB];

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

  // Q^T as the B operand: lane holds Q[q0 + 16 qt + c16][32 ks + 8 g4 + 0..7].
  op8 qf[QT][KS];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int q = q0 + 16 * qt + c16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (q < R) v = *(const u32x4*)(base + (size_t)q * ld + (size_t)h * HD + 32 * ks + 8 * g4);
      qf[qt][ks] = __builtin_bit_cast(op8, v);
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
  // QPRE (Q already scaled): the score MFMAs start from c0 = -mref, so they
  // yield the exponent itself, and mref starts at block 0's row maxima;
  // otherwise mref starts at -inf and every score takes one FMA.
  float mref[QT];
  f32x4 osum[QT], c0[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    mref[qt] = QPRE ? 0.f : -INFINITY;
    osum[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
    c0[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const uint32_t one2 = c16 == 0 ? H::one2 : 0u;   // two ones, or zeros
  const op8 ones_row = __builtin_bit_cast(op8, u32x4{one2, one2, one2, one2});

  // K/V block loads straight into LDS: wave-wide load q of a block moves
  // 1 KiB, rows RPL q .. RPL q + RPL - 1, lane L landing at byte 16 L, i.e.
  // row RPL q + L / CPR at physical chunk L % CPR, which holds that row's
  // logical chunk (L % CPR) ^ swz(row).  The buffer resource starts at the
  // block's first row and ends with the cell, so keys past R read as zeros
  // (their scores are masked, and zero V rows keep P V finite).  Per-lane
  // offsets are the same for every block.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  __builtin_assume(wave_u >= 0 && wave_u < 4);
  // K and V share the row permutation, so a V load is its K load moved by the
  // uniform Hkv * HD columns (the buffer's scalar offset).
  int koff[PPW];
#pragma unroll
  for (int i = 0; i < PPW; ++i) {
    const int row = RPL * (wave_u + 4 * i) + lane / CPR;
    koff[i] = (row * ld + (Hq + kvh) * HD + 8 * ((lane % CPR) ^ swz<HD>(row))) * 2;
  }
  const int vdelta = Hkv * HD * 2;
  auto fetch = [&](int kb, int slot) __attribute__((always_inline)) {
    const int k0 = kb * KB;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(base + (size_t)k0 * ld), (short)0, (R - k0) * ld * 2, BUF_FLAGS);
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
      const int q = wave_u + 4 * i;
      load_lds16(rs, &sK[slot][q * 1024], koff[i], 0);
      load_lds16(rs, &sV[slot][q * 1024], koff[i], vdelta);
    }
  };
  // Every wave waits for its own loads into LDS, then a bare barrier makes
  // the block visible to the workgroup (and certifies that the other slot's
  // readers are done).  The empty asm statements keep LDS accesses on their
  // side of it.
  auto block_sync = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt((7 << 4) | (0 << 8));   // vmcnt(0) lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // keys needed by any of the workgroup's query rows: [0, kend)
  const int kend = CAUSAL ? min(qg0 + qw * QB, R) : R;
  const int nkb = (kend + KB - 1) / KB;
  // The K rows a lane reads are 16 kt + c16, whose permutation is that of c16.
  const int kswz = swz<HD>(c16);
  // S^T block: 64 keys x QB queries.  Lane holds keys 16 kt + 4 g4 + j of
  // query column 16 qt + c16: raw scores, or with QPRE scaled scores minus
  // mref (the accumulation starts from c0).  Then the masked scores: keys
  // past the cell's end and, when causal, keys after the query.  (A causal
  // block wholly after this wave's rows masks them all: its probabilities
  // are exactly zero.)
  auto scores = [&](const uint8_t* K_, int k0, f32x4 (&s)[4][QT]) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const op8 kf = __builtin_bit_cast(
            op8, *(const u32x4*)(K_ + (16 * kt + c16) * ROWB + 16 * ((4 * ks + g4) ^ kswz)));
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          s[kt][qt] = H::mfma(kf, qf[qt][ks], ks == 0 ? c0[qt] : s[kt][qt]);
      }
    if ((CAUSAL && k0 + KB - 1 > q0) || (k0 + KB > R)) {   // wave-uniform
      // element (kt, j) holds key k0 + 16 kt + 4 g4 + j: it is masked when
      // 16 kt + j exceeds a limit that depends on the lane and the query tile
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const int last = CAUSAL ? min(q0 + 16 * qt + c16, R - 1) : R - 1;   // last visible key
        const int lim = last - k0 - 4 * g4;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (16 * kt + j > lim) s[kt][qt][j] = -INFINITY;
      }
    }
  };
  fetch(0, 0);
  block_sync();
  if constexpr (QPRE) {
    // The reference maxima come from block 0, which every row sees (key 0 is
    // visible to all): its scores are formed once more inside the loop, then
    // relative to this reference.
    f32x4 s[4][QT];
    scores(sK[0], 0, s);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        mx = fmaxf(fmaxf(mx, s[kt][qt][0]), s[kt][qt][1]);
        mx = fmaxf(fmaxf(mx, s[kt][qt][2]), s[kt][qt][3]);
      }
      mref[qt] = max_over_groups(mx);
      c0[qt] = f32x4{-mref[qt], -mref[qt], -mref[qt], -mref[qt]};
    }
  }
  for (int kb = 0; kb < nkb; ++kb) {
    const int slot = kb & 1;
    const int k0 = kb * KB;
    if (kb + 1 < nkb) fetch(kb + 1, slot ^ 1);
    const uint8_t* K_ = sK[slot];
    const uint8_t* V_ = sV[slot];

    f32x4 s[4][QT];
    scores(K_, k0, s);

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
      if constexpr (QPRE) need_rescale |= mx > RESCALE_LOG2;
      else need_rescale |= mx * scale_log2 > mref[qt] + RESCALE_LOG2;
    }
    if constexpr (QPRE) {
      // A rescale moves the reference up by what the row maximum exceeds it
      // and the block's exponents down by the same amount.
      if (__any(need_rescale)) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          const float shift = fmaxf(max_over_groups(mloc[qt]), 0.f);
          const float corr = __builtin_amdgcn_exp2f(-shift);
          osum[qt] *= corr;
#pragma unroll
          for (int ht = 0; ht < HT; ++ht) o[ht][qt] *= corr;
          mref[qt] += shift;
          c0[qt] = f32x4{-mref[qt], -mref[qt], -mref[qt], -mref[qt]};
#pragma unroll
          for (int kt = 0; kt < 4; ++kt) s[kt][qt] -= shift;
        }
      }
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int j = 0; j < 4; ++j) s[kt][qt][j] = __builtin_amdgcn_exp2f(s[kt][qt][j]);
    } else {
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
    }

    // O^T += V^T P^T over two 32-key steps.  In step ks2, operand slot e < 4
    // is key 32 ks2 + 4 g4 + e and slot e >= 4 is key 32 ks2 + 16 + 4 g4 +
    // (e - 4), matching where the S^T accumulator left those probabilities.
    // The transposing read: lane j of each 16-lane group points at row
    // key0 + j / 4, columns 4 (j % 4) .. +3; lane i receives column i of the
    // four rows.
    const int tr_row = 4 * g4 + (c16 >> 2);
    const int tr_chunk = (c16 & 3) >> 1;     // columns 4 (c16 & 3) .. +3: chunk and byte in it
    const int tr_byte = 8 * (c16 & 1);
    const int vswz = swz<HD>(tr_row);        // rows 32 ks2 + tr_row (+ 16): same permutation
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      op8 pf[QT];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        u32x4 w;
        w[0] = H::pack(s[2 * ks2][qt][0], s[2 * ks2][qt][1]);
        w[1] = H::pack(s[2 * ks2][qt][2], s[2 * ks2][qt][3]);
        w[2] = H::pack(s[2 * ks2 + 1][qt][0], s[2 * ks2 + 1][qt][1]);
        w[3] = H::pack(s[2 * ks2 + 1][qt][2], s[2 * ks2 + 1][qt][3]);
        pf[qt] = __builtin_bit_cast(op8, w);
        osum[qt] = H::mfma(ones_row, pf[qt], osum[qt]);
      }
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        const uint8_t* v0 = V_ + (32 * ks2 + tr_row) * ROWB + 16 * ((2 * ht + tr_chunk) ^ vswz) + tr_byte;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(v0));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(v0 + 16 * ROWB));
        u32x4 w;
        const u32x2 wl = __builtin_bit_cast(u32x2, lo);
        const u32x2 wh = __builtin_bit_cast(u32x2, hi);
        w[0] = wl[0];
        w[1] = wl[1];
        w[2] = wh[0];
        w[3] = wh[1];
        const op8 vf = __builtin_bit_cast(op8, w);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          o[ht][qt] = H::mfma(vf, pf[qt], o[ht][qt]);
      }
    }

    block_sync();
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
      w[0] = H::pack(o[ht][qt][0] * inv, o[ht][qt][1] * inv);
      w[1] = H::pack(o[ht][qt][2] * inv, o[ht][qt][3] * inv);
      *(u32x2*)(orow + 16 * ht + 4 * g4) = w;
    }
  }
}

}  // namespace

hipError_t launch_attention(const uint16_t* qkv, uint16_t* out, int G, int R, int Hq, int Hkv,
                            int hd, bool causal, bool q_prescaled, hipStream_t stream, bool f16) {
  if (G == 0 || R == 0) return hipSuccess;
  if (Hkv < 1 || Hq < 1 || R < 0 || Hq % Hkv != 0) return hipErrorInvalidValue;
  const int rep = Hq / Hkv;
  if (!(rep == 1 || rep == 2 || rep % 4 == 0)) return hipErrorInvalidValue;
  // K/V loads address one cell's rows with 32-bit buffer offsets
  if ((size_t)R * (size_t)(Hq + 2 * Hkv) * (size_t)hd * 2 > (size_t)INT32_MAX) return hipErrorInvalidValue;
  if (f16 && !(causal && q_prescaled)) return hipErrorInvalidValue;   // fp16: the LLaMA cell's stage only
  const float scale_log2 = attention_scale_log2(hd);
  constexpr int QB = 32;   // measured faster than 64: lower register use, more waves
  const int hw = rep >= 4 ? 4 : rep;
  const int qw = 4 / hw;
  const int nqb = (R + QB - 1) / QB;
  const dim3 grid((nqb + qw - 1) / qw, Hkv * (rep / hw), G);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, qkv, out, R, Hq, Hkv, scale_log2);
  };
  if (hd == 64) {
    if (f16) go(attention_kernel<64, QB, true, true, true>);
    else if (q_prescaled) {
      if (causal) go(attention_kernel<64, QB, true, true, false>);
      else go(attention_kernel<64, QB, false, true, false>);
    } else {
      if (causal) go(attention_kernel<64, QB, true, false, false>);
      else go(attention_kernel<64, QB, false, false, false>);
    }
  } else if (hd == 128) {
    if (f16) go(attention_kernel<128, QB, true, true, true>);
    else if (q_prescaled) {
      if (causal) go(attention_kernel<128, QB, true, true, false>);
      else go(attention_kernel<128, QB, false, true, false>);
    } else {
      if (causal) go(attention_kernel<128, QB, true, false, false>);
      else go(attention_kernel<128, QB, false, false, false>);
    }
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rmt
