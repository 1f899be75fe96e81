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
// Design (measured on MI355X: no one unit saturates.  The operand stream into
// LDS, the LDS reads -- conflict free, 4 LDS cycles per 16-byte wave read,
// with waves waiting to issue them 2-3% of their cycles -- and the MFMAs each
// run well below their rates, and with every operand L2-resident the kernel
// runs no faster.  What binds is each slice's barrier across the workgroup's
// waves under the chip's power limit, so tiles are as large as LDS and the
// register file allow):
//   * Output tiles of 288, 256, 192 or 128 rows x 256 columns, chosen per launch
//     by a cost model of whole rounds of one tile per CU (see launch_epi);
//     waves compute 32 x 32 blocks with v_mfma_f32_32x32x16_bf16.  A cell
//     (group) never shares a tile with another; the rows past the cell's end
//     read as zeros and waves that own only such rows skip their MFMAs.
//   * K advances 64 at a time through a two-slice LDS ring filled by buffer
//     loads that write LDS directly (no staging registers).  LDS rows are
//     unpadded; their 16-byte chunks are XOR-swizzled so MFMA operand reads
//     of 32 consecutive rows are bank-conflict free.  Buffer resources clip
//     every load to the tile's valid rows and K, so ragged edges are zeros
//     without branches.
//   * Workgroup ids are renumbered so each XCD (ids = x mod 8) receives a
//     contiguous run of tiles; within a cell the M tile varies fastest, so the
//     tiles sharing a weight panel run together in one XCD's L2.
//   * Epilogues fuse what follows each product in the cell: RoPE and the
//     softmax scale (QKV), SwiGLU (gate/up), biases and ReLU, the fp32
//     residual add with the split write-back of X and M rows, and for the
//     LLaMA-shaped cell the next RMSNorm's inputs (the 16-bit copy y * gamma
//     and 64-column chunk sums of y^2) and the 1/rms row scales of its
//     consumers.
//   * Every output element is produced by one lane with the same K order for
//     every tile shape and every G, so a cell's result does not depend on
//     which diagonal (or the sequential sweep) it runs in.
#include "kernels.h"

#include <type_traits>

namespace rmt {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BN = 256;
constexpr int BK = 64;
constexpr int STAGES = 2;
constexpr int ROWB = BK * 2;         // bytes per LDS row: unpadded, chunks XOR-swizzled
constexpr int CPR = BK / 8;          // 16-byte chunks per row
constexpr int RPI = 64 / CPR;        // rows filled by one wave-wide 1 KiB load
constexpr int BUF_FLAGS = 0x00020000;        // raw buffer, 32-bit data format

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// The 16-bit type of a launch's operands and 16-bit results: bf16, or IEEE
// half (fp16: three more mantissa bits, the same MFMA rate).  `pack` turns
// two fp32 values into the packed pair, rounding to nearest even
// (v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32).
template <bool F16>
struct Half16 {
  typedef __bf16 x8 __attribute__((ext_vector_type(8)));
  typedef __bf16 x2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ f32x16 mfma(x8 a, x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
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
  static __device__ __forceinline__ f32x16 mfma(x8 a, x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    x2 v;
    v[0] = (_Float16)lo;
    v[1] = (_Float16)hi;
    return __builtin_bit_cast(uint32_t, v);
  }
};

// Chunk permutation of LDS row r: logical 16-byte chunk c sits at physical
// position c ^ swz(r).  It depends only on r mod 32, and 16-byte reads of 32
// consecutive rows at one logical chunk are free of bank conflicts on gfx950:
// measured, both by a probe of this read pattern (4 LDS cycles per wave-wide
// read, the conflict-free rate) and by the kernel's own bank-conflict counter.
__device__ __forceinline__ int swz(int r) {
  if constexpr (CPR == 8) return ((r >> 1) ^ ((r & 1) << 2)) & 7;
  else return ((r >> 1) + (r >> 3)) & 3;
}

// s_waitcnt that leaves at most N vector-memory operations outstanding and
// none of this wave's LDS reads (so no stage is refilled under a reader).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N < 64, "vmcnt has 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}

// Global-memory pointers (address space 1), so that stores through them stay
// global stores rather than flat ones (flat stores also count against the
// LDS wait counter).
typedef __attribute__((address_space(1))) uint16_t gu16;
typedef __attribute__((address_space(1))) float gf32;
typedef __attribute__((address_space(1))) u32x2 gu32x2;
typedef __attribute__((address_space(1))) f32x4 gf32x4;

// A pointer that is the same in every lane, moved to scalar registers.
template <typename T>
__device__ __forceinline__ T* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (T*)(((uint64_t)hi << 32) | lo);
}

// Workgroups are handed to the 8 XCDs round-robin (id mod 8).  Renumber them
// so that each XCD receives one contiguous run of tiles: tiles that share a
// weight panel then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int nb) {
  const int per = nb >> 3, rem = nb & 7;
  const int xcd = bid & 7, idx = bid >> 3;
  return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

// BM x BN output tile per workgroup; WTM x WTN is one wave's sub-tile and the
// workgroup has one wave per sub-tile.
// BNT: weight slices are loaded with the non-temporal policy (see launch_one).
// F16: operands and 16-bit results in fp16 instead of bf16.
template <int EPI, int BM, int WTM, int WTN, bool BNT, bool F16>
__global__ __launch_bounds__((BM / WTM) * (BN / WTN) * 64, 1) void gemm_bf16_kernel(
    GemmArgs a, GroupTable tab, NormAux aux) {
  using H = Half16<F16>;
  typedef typename H::x8 op8;
  constexpr int STAGE_BYTES = (BM + BN) * ROWB;
  // The MFMAs take the operands swapped, so the accumulator holds C^T blocks
  // and every lane owns four consecutive output columns of one row: the
  // epilogues then move 8- and 16-byte vectors instead of single elements.
  constexpr bool SWAP = true;
  constexpr int WAVES_N = BN / WTN;
  constexpr int NWAVES = (BM / WTM) * WAVES_N;
  constexpr int MI = WTM / 32;
  constexpr int NI = WTN / 32;
  // The (BM + BN) / RPI wave-wide loads of a K slice are dealt round-robin
  // to the waves; the count per wave differs by at most one.
  constexpr int A_LOADS = BM / RPI;
  constexpr int ALL_LOADS = (BM + BN) / RPI;
  constexpr int LOADS_PER_WAVE = (ALL_LOADS + NWAVES - 1) / NWAVES;
  static_assert(A_LOADS * RPI == BM && ALL_LOADS * RPI == BM + BN, "load split");
  // vmcnt-based waits for slices still in flight need the same count per wave
  static_assert(STAGES == 2 || ALL_LOADS % NWAVES == 0, "uneven load split needs a two-slice ring");
  constexpr bool SIDE = EPI == EPI_RESID_NORM_F32;   // RMSNorm side outputs
  // One LDS array for everything.  A second __shared__ object makes the
  // compiler tag LDS accesses with alias scopes, and it then drains every
  // in-flight direct-to-LDS load before the first LDS read of each K slice,
  // which serialises the ring; the waits below already order the slices.
  constexpr int GSM_OFF = STAGES * STAGE_BYTES;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[GSM_OFF + (SIDE ? 2 * BN * 4 : 0)];
  // side outputs: the tile's gains for its lo rows ([0, BN)) and hi rows
  float* const gsm = (float*)(smem + GSM_OFF);

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
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;

  const int K = a.K;
  const int m_valid = min(BM, a.M - tm * BM);
  const int n_valid = min(BN, a.N - tn * BN);
  // Buffer resources clipped to the tile's valid rows: the hardware returns
  // zeros for anything outside, so ragged M / N / K edges need no branches.
  const uint16_t* Bg = a.B + ((size_t)tab.layer[g] * a.N + (size_t)tn * BN) * K;
  const int a_bytes = m_valid * K * 2;
  const int b_bytes = n_valid * K * 2;
  // A split (QKV of the LLaMA cell): the tile's rows below a_split come from
  // in_lo[g] (the cell's memory rows), the others from in_hi[g] (its segment
  // rows).  ra covers the lo rows of the tile, ra_hi all of its rows as they
  // sit in in_hi (the rows below a_split are never read through it, so its
  // base may point before in_hi).  Each wave-wide load spans 8 rows and
  // a_split is a multiple of 8, so a load lies wholly in one part.
  constexpr bool SPLIT_A = EPI == EPI_QKV_ROPE;
  const bool split_a = SPLIT_A && a.a_split > 0;
  __amdgpu_buffer_rsrc_t ra, ra_hi;
  if (split_a) {
    const int lo_rows = max(0, min(m_valid, a.a_split - tm * BM));
    const uint16_t* lo = (const uint16_t*)tab.in_lo[g] + (size_t)tm * BM * K;
    const uintptr_t hi = (uintptr_t)tab.in_hi[g] + (intptr_t)(tm * BM - a.a_split) * K * 2;
    ra = __builtin_amdgcn_make_buffer_rsrc((void*)lo, (short)0, lo_rows * K * 2, BUF_FLAGS);
    ra_hi = __builtin_amdgcn_make_buffer_rsrc((void*)hi, (short)0, a_bytes, BUF_FLAGS);
  } else {
    const uint16_t* Ag = a.A + ((size_t)g * a.M + (size_t)tm * BM) * K;
    ra = __builtin_amdgcn_make_buffer_rsrc((void*)Ag, (short)0, a_bytes, BUF_FLAGS);
    ra_hi = ra;
  }
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc((void*)Bg, (short)0, b_bytes, BUF_FLAGS);

  // Global -> LDS without registers: each wave-wide load moves 1 KiB, lane L
  // landing at byte 16 L of the destination, i.e. row RPI q + L / CPR at
  // physical chunk L % CPR, which holds logical chunk (L % CPR) ^ swz(row).
  const int lrow = lane / CPR;
  const int lp = lane % CPR;
  // Per-lane byte offsets of this wave's loads at k = 0 (loop invariant); a
  // K slice adds 2 k0 to them.  The wave index is taken as a uniform value so
  // that the LDS destination (M0) is computed with scalar instructions.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  __builtin_assume(wave_u >= 0 && wave_u < NWAVES);
  int koff[LOADS_PER_WAVE];
#pragma unroll
  for (int i = 0; i < LOADS_PER_WAVE; ++i) {
    const int q = min(wave_u + i * NWAVES, ALL_LOADS - 1);
    const bool is_a = q < A_LOADS;
    const int row = (is_a ? q : q - A_LOADS) * RPI + lrow;
    koff[i] = (row * K + 8 * (lp ^ swz(row))) * 2;
  }
  const bool k_whole = K % BK == 0;
  // CHECKED: the partial last K slice, whose columns past K must read as
  // zeros (their offsets are moved past the end of the buffer).
  auto issue_slice = [&](int kt, int stage, auto checked_c) __attribute__((always_inline)) {
    constexpr bool CHECKED = decltype(checked_c)::value;
    const int k0 = kt * BK;
    uint8_t* sbase = smem + stage * STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < LOADS_PER_WAVE; ++i) {
      const int q = wave_u + i * NWAVES;        // wave-uniform
      if (ALL_LOADS % NWAVES != 0 && q >= ALL_LOADS) break;
      // i is a constant after unrolling: the operand is known at compile time
      // unless the A/B boundary falls inside this round of loads
      const bool is_a = (i + 1) * NWAVES <= A_LOADS ? true : i * NWAVES >= A_LOADS ? false : q < A_LOADS;
      int off = koff[i] + 2 * k0;
      if constexpr (CHECKED) {
        const int row = (is_a ? q : q - A_LOADS) * RPI + lrow;
        if (k0 + 8 * (lp ^ swz(row)) >= K) off = is_a ? a_bytes : b_bytes;
      }
      // rows of load q start at tm * BM + q * RPI (wave-uniform)
      const __amdgpu_buffer_rsrc_t rsa = SPLIT_A && tm * BM + q * RPI >= a.a_split ? ra_hi : ra;
      if constexpr (BNT) {
        if (is_a) __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_ptr_t)(sbase + q * 1024), 16, off, 0, 0, 0);
        else __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(sbase + q * 1024), 16, off, 0, 0, 2);
      } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(is_a ? rsa : rb, (lds_ptr_t)(sbase + q * 1024), 16, off, 0, 0, 0);
      }
    }
  };
  auto issue = [&](int kt, int stage) __attribute__((always_inline)) {
    if (!k_whole && kt == (K - 1) / BK) issue_slice(kt, stage, std::true_type{});
    else issue_slice(kt, stage, std::false_type{});
  };

  f32x16 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int t = 0; t < NI; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][t][e] = 0.f;

  // Lane l feeds row (l % 32) of its A/B blocks with 8 consecutive k values.
  // Within one K slice lanes 0-31 cover the first half of the slice and lanes
  // 32-63 the second half, over the slice's MFMA steps; A and B use the same
  // assignment, so each MFMA still sums matching k.
  // A wave whose rows all lie past the tile's valid rows (the short last
  // tile of a cell) has nothing to compute; it still loads and synchronises.
  const bool wave_live = wm * WTM < m_valid;
  const int r32 = lane & 31;
  const int sw = swz(r32);             // == swz of every row this lane reads
  const int c0 = (lane >> 5) * (CPR / 2);
  const int a_row = (wm * WTM + r32) * ROWB;
  const int b_row = BM * ROWB + (wn * WTN + r32) * ROWB;
  auto compute = [&](int stage) __attribute__((always_inline)) {
    const uint8_t* sbase = smem + stage * STAGE_BYTES;
    op8 af[2][MI], bfr[2][NI];
    auto frags = [&](int j, int buf) __attribute__((always_inline)) {
      const int cb = ((c0 + j) ^ sw) * 16;
#pragma unroll
      for (int i = 0; i < MI; ++i)
        af[buf][i] = __builtin_bit_cast(op8, *(const u32x4*)(sbase + a_row + i * 32 * ROWB + cb));
#pragma unroll
      for (int t = 0; t < NI; ++t)
        bfr[buf][t] = __builtin_bit_cast(op8, *(const u32x4*)(sbase + b_row + t * 32 * ROWB + cb));
    };
    frags(0, 0);
#pragma unroll
    for (int j = 0; j < CPR / 2; ++j) {
      if (j + 1 < CPR / 2) frags(j + 1, (j + 1) & 1);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int t = 0; t < NI; ++t)
          if constexpr (SWAP)
            acc[i][t] = H::mfma(bfr[j & 1][t], af[j & 1][i], acc[i][t]);
          else
            acc[i][t] = H::mfma(af[j & 1][i], bfr[j & 1][t], acc[i][t]);
      // let the scheduler interleave LDS reads with the MFMA chain
      __builtin_amdgcn_iglp_opt(1);
    }
  };

  // Row scales (an RMSNorm's 1/rms per output row) are requested now and
  // applied to the accumulators after the main loop.
  constexpr bool ROWSCALE = EPI == EPI_QKV_ROPE || EPI == EPI_SWIGLU;
  float rsc[ROWSCALE ? MI : 1];
  if constexpr (ROWSCALE) {
    if (a.row_scale) {
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int row = tm * BM + wm * WTM + i * 32 + r32;
        rsc[i] = row < a.M ? a.row_scale[(size_t)g * a.M + row] : 0.f;
      }
    }
  }
  // Side-output gains of the tile's columns, for its lo and hi rows, into LDS
  // beside the ring (the main loop's first barrier publishes them).
  if constexpr (SIDE) {
    for (int j = tid; j < 2 * BN; j += NWAVES * 64) {
      const int part = j / BN, c = j % BN, col = tn * BN + c;
      const int lay = part ? aux.layer_hi[g] : aux.layer_lo[g];
      gsm[part * BN + c] = col < a.N ? a.aux_gamma[(size_t)lay * a.N + col] : 0.f;
    }
  }

  // Ring of STAGES LDS slices: slice kt+STAGES-1 is requested while the
  // MFMAs consume slice kt.  One barrier per slice; it also certifies that
  // every wave has finished reading the stage about to be refilled.
  const int nk = (K + BK - 1) / BK;
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nk) issue(s, s);
  for (int kt = 0; kt < nk; ++kt) {
    const int ahead = min(nk - 1 - kt, STAGES - 2);   // later slices still in flight
    if (ahead == 0) wait_vmem<0>();
    else wait_vmem<LOADS_PER_WAVE>();
    // Each wave has waited for its own LDS-bound loads above; a bare barrier
    // (no release fence, which would drain every load still in flight) makes
    // them visible to the whole workgroup.  The empty asm statements keep the
    // compiler from moving LDS accesses across it.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kt + STAGES - 1 < nk) issue(kt + STAGES - 1, (kt + STAGES - 1) % STAGES);
    if (wave_live) compute(kt % STAGES);
  }

  // ---- Epilogue ----
  // Accumulator layout (C^T blocks): element e of lane l of block (i, t) is
  // row i*32 + l%32, column t*32 + 8*(e/4) + 4*(l/32) + e%4.  A wave-wide
  // access straight from that layout touches 32 rows at 16-32 bytes each, so
  // the bf16 epilogues go through a private LDS region of the wave and read
  // it back row-major, so that their stores cover whole row segments: the
  // plain-store, bias and SwiGLU epilogues finish their arithmetic on the
  // accumulators and stage bf16 results; RoPE stages the two fp32 blocks of
  // a rotation pair and rotates after the read-back.  The fp32 residual
  // epilogues work straight from the accumulator layout.
  if constexpr (ROWSCALE) {
    if (a.row_scale) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int t = 0; t < NI; ++t) acc[i][t] *= rsc[i];
    }
  }
  constexpr bool RESID = EPI == EPI_RESID_F32 || EPI == EPI_RESID_BIAS_F32 || SIDE;
  if constexpr (!RESID || SIDE) {   // SIDE stages its 16-bit copies through the ring
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();      // the ring is free once every wave is past its last slice
    asm volatile("" ::: "memory");
  }
  constexpr int EP_LD = 68;            // floats per staged row: 64 + 4 of padding
  static_assert(NWAVES * 32 * EP_LD * 4 <= STAGES * STAGE_BYTES, "epilogue staging fits the ring");
  static_assert(NI % 2 == 0, "pieces are pairs of 32-column blocks");
  float* ep = (float*)smem + wave * 32 * EP_LD;
  const int wrow0 = tm * BM + wm * WTM;        // first row of the wave's sub-tile
  const int wcol0 = tn * BN + wn * WTN;        // first column of the wave's sub-tile
  const int half_lane = 4 * (lane >> 5);

  // Wave-local LDS hand-off: all of this wave's LDS accesses issued so far
  // have completed, and the compiler keeps later ones after this point.
  auto lds_sync = [&]() __attribute__((always_inline)) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };
  // Block (i, t) of the accumulator -> columns [32 slot, 32 slot + 32) of the piece.
  auto stage = [&](const f32x16& blk, int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4)
      *(f32x4*)(ep + r32 * EP_LD + slot * 32 + 8 * e4 + half_lane) =
          f32x4{blk[4 * e4], blk[4 * e4 + 1], blk[4 * e4 + 2], blk[4 * e4 + 3]};
  };

  if constexpr (RESID) {
    // The group's side-output pointers, read once as wave-uniform values (a
    // per-lane choice between the table's entries would otherwise become a
    // per-lane load from the argument block inside every row block).
    gu16* aux_rows_lo = nullptr;
    gu16* aux_rows_hi = nullptr;
    gf32* aux_ss_lo = nullptr;
    gf32* aux_ss_hi = nullptr;
    if constexpr (SIDE) {
      aux_rows_lo = uniform_ptr<gu16>(aux.rows_lo[g]);
      aux_rows_hi = uniform_ptr<gu16>(aux.rows_hi[g]);
      aux_ss_lo = uniform_ptr<gf32>(aux.ss_lo[g]);
      aux_ss_hi = uniform_ptr<gf32>(aux.ss_hi[g]);
    }
    // Straight from the accumulator layout.  All residual loads of a 32-row
    // block are issued before any of its stores: the compiler cannot prove
    // that `out` does not alias `res`, and would otherwise wait out one full
    // memory round trip per load.  The group's row pointers are read once as
    // wave-uniform values and chosen per lane by value (choosing between
    // table entries per lane would load the pointer per lane, in every row
    // block, before the residual loads could start).
    const gf32* res_lo = uniform_ptr<const gf32>(tab.in_lo[g]);
    const gf32* res_hi = uniform_ptr<const gf32>(tab.in_hi[g]);
    gf32* out_lo = uniform_ptr<gf32>(tab.out_lo[g]);
    gf32* out_hi = uniform_ptr<gf32>(tab.out_hi[g]);
    constexpr bool BIAS_R = EPI == EPI_RESID_BIAS_F32;
    const gf32* bias_l = BIAS_R ? (const gf32*)(a.bias + (size_t)tab.layer[g] * a.N) : nullptr;
    // The code below is straight-line per 32-row block: column validity is
    // decided per 32-column block (N is a multiple of 32 on these paths,
    // checked at launch), which is the same for the whole wave, and every
    // side output has a destination.  Per-lane branches here would leave the
    // compiler's wait counting no choice but to drain every store before each
    // of the next stores' residuals is used.
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      // Every lane stays active (the staged read-back below hands rows to
      // other lanes): rows past M load from the last valid row and store
      // nothing.
      const int row_t = wrow0 + i * 32 + r32;
      const bool row_ok = row_t < a.M;
      const int row = row_ok ? row_t : a.M - 1;
      const gf32* res = row < a.split_in ? res_lo + (size_t)row * a.ld_res
                                         : res_hi + (size_t)(row - a.split_in) * a.ld_res;
      gf32* out = row < a.split_out ? out_lo + (size_t)row * a.ld_out
                                    : out_hi + (size_t)(row - a.split_out) * a.ld_out;
      f32x4 rv[NI][4];
#pragma unroll
      for (int t = 0; t < NI; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = wcol0 + t * 32 + 8 * q + half_lane;
          rv[t][q] = wcol0 + t * 32 < a.N ? *(const gf32x4*)(res + col) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
      // The bias (EPI_RESID_BIAS_F32) is loaded again for every row block, a
      // cache hit after the first: kept live across the row blocks, its
      // vectors would be spilled.
      f32x4 bv[BIAS_R ? NI : 1][4];
      if constexpr (BIAS_R) {
#pragma unroll
        for (int t = 0; t < NI; ++t)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = wcol0 + t * 32 + 8 * q + half_lane;
            bv[t][q] = wcol0 + t * 32 < a.N ? *(const gf32x4*)(bias_l + col) : f32x4{0.f, 0.f, 0.f, 0.f};
          }
      }
      // y = residual + acc (+ bias: residual + (acc + bias)) in rv, then the
      // fp32 stores of the row block
#pragma unroll
      for (int t = 0; t < NI; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if constexpr (BIAS_R) rv[t][q][e] += acc[i][t][4 * q + e] + bv[t][q][e];
            else rv[t][q][e] += acc[i][t][4 * q + e];
          }
      if (row_ok) {
#pragma unroll
        for (int t = 0; t < NI; ++t) {
          if (wcol0 + t * 32 >= a.N) break;      // wave-uniform
#pragma unroll
          for (int q = 0; q < 4; ++q) *(gf32x4*)(out + wcol0 + t * 32 + 8 * q + half_lane) = rv[t][q];
        }
      }
      if constexpr (SIDE) {
        // Side outputs (EPI_RESID_NORM_F32).  The 64-column chunk sums: both
        // half-lanes of a row add their 32 squares, in the same order, and
        // store the same value to the same place.  The 16-bit copies y * g go
        // through the wave's LDS region (32 rows of WTN values, 16-byte chunks
        // XOR-swizzled by row) and leave as row segments, 8 rows of WTN * 2
        // bytes per store, like the bf16 epilogues' results.
        const bool lo_part = row < a.split_out;
        const int rr_own = lo_part ? row : row - a.split_out;
        gf32* xss = (lo_part ? aux_ss_lo : aux_ss_hi) + rr_own;
        const int ss_ld = lo_part ? aux.ss_ld_lo : aux.ss_ld_hi;
        constexpr int OCH = WTN / 8;
        auto swz_s = [](int r) { return OCH == 8 ? ((r >> 1) & 7) : (r & (OCH - 1)); };
        uint16_t* sp = (uint16_t*)(smem + wave * 32 * WTN * 2);
        float chunk_ss = 0.f;
#pragma unroll
        for (int t = 0; t < NI; ++t) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4 r = rv[t][q];
            const int col = wcol0 + t * 32 + 8 * q + half_lane;
            chunk_ss += (r[0] * r[0] + r[1] * r[1]) + (r[2] * r[2] + r[3] * r[3]);
            const f32x4 gw = *(const f32x4*)&gsm[(lo_part ? 0 : BN) + col - tn * BN];
            const int c = (t * 4 + q) ^ swz_s(r32);
            *(u32x2*)(sp + r32 * WTN + c * 8 + half_lane) =
                u32x2{H::pack(r[0] * gw[0], r[1] * gw[1]), H::pack(r[2] * gw[2], r[3] * gw[3])};
          }
          if (t & 1) {
            const float other = __shfl_xor(chunk_ss, 32);
            const float tot = lane < 32 ? chunk_ss + other : other + chunk_ss;
            if (row_ok && wcol0 + t * 32 < a.N)
              __builtin_nontemporal_store(tot, xss + (size_t)((wcol0 + t * 32) / kChunk) * ss_ld);
            chunk_ss = 0.f;
          }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        // read back row-major: OCH lanes per staged row, 64 / OCH rows per
        // access; each row's part decides its destination
        const int rc = lane % OCH;
        const int ocol = wcol0 + rc * 8;
#pragma unroll
        for (int k = 0; k < 32 * OCH / 64; ++k) {
          const int rr = k * (64 / OCH) + lane / OCH;
          const u32x4 v = *(const u32x4*)(sp + rr * WTN + (rc ^ swz_s(rr)) * 8);
          const int orow = wrow0 + i * 32 + rr;
          if (orow < a.M && ocol < a.N) {
            gu16* dst = orow < a.split_out ? aux_rows_lo + (size_t)orow * a.N
                                           : aux_rows_hi + (size_t)(orow - a.split_out) * a.N;
            // non-temporal: read two launches later, not by this one's tiles
            __builtin_nontemporal_store(v, (__attribute__((address_space(1))) u32x4*)(dst + ocol));
          }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      }
    }
  } else if constexpr (EPI == EPI_STORE_BF16 || EPI == EPI_BIAS_BF16 || EPI == EPI_BIAS_RELU_BF16) {
    // Bias and ReLU run on the accumulators (a lane's four consecutive
    // columns share one 16-byte bias load, the same for every row block);
    // each 32-row block of the wave's outputs is then staged as bf16 -- rows
    // of WTN values whose 16-byte chunks are XOR-swizzled, so the staging
    // writes of 32 rows spread over the banks -- and read back row-major for
    // 16-byte stores.  Output columns come in whole 8-column chunks (the host
    // requires N % 8 == 0).
    constexpr bool BIAS = EPI != EPI_STORE_BF16;
    constexpr int OCH = WTN / 8;                  // 16-byte chunks per staged row
    static_assert(32 * WTN * 2 <= 32 * EP_LD * 4, "a staged row block fits the wave's region");
    auto swz_o = [](int r) { return OCH == 8 ? ((r >> 1) & 7) : (r & (OCH - 1)); };
    uint16_t* sp = (uint16_t*)ep;
    uint16_t* C = (uint16_t*)tab.out_lo[g];
    f32x4 bv[BIAS ? NI : 1][4];
    if constexpr (BIAS) {
      const float* bl = a.bias + (size_t)tab.layer[g] * a.N;
#pragma unroll
      for (int t = 0; t < NI; ++t)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int col = wcol0 + t * 32 + 8 * e4 + half_lane;
          bv[t][e4] = col < a.N ? *(const f32x4*)(bl + col) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    // Q columns of the QKV projection take the attention scale (a 32-column
    // block is wholly Q or not; 1.0 elsewhere leaves the values unchanged).
    float qs[NI];
#pragma unroll
    for (int t = 0; t < NI; ++t) qs[t] = wcol0 + t * 32 < a.q_cols ? a.q_scale : 1.0f;
    const int rc = lane % OCH;
    const int col = wcol0 + rc * 8;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
      for (int t = 0; t < NI; ++t)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          f32x4 x = {acc[i][t][4 * e4], acc[i][t][4 * e4 + 1], acc[i][t][4 * e4 + 2], acc[i][t][4 * e4 + 3]};
          if constexpr (BIAS) {
            x += bv[t][e4];
            if constexpr (EPI == EPI_BIAS_RELU_BF16) {
#pragma unroll
              for (int e = 0; e < 4; ++e) x[e] = fmaxf(x[e], 0.f);
            }
          }
          if constexpr (EPI == EPI_BIAS_BF16) x *= qs[t];
          const int c = (t * 4 + e4) ^ swz_o(r32);
          *(u32x2*)(sp + r32 * WTN + c * 8 + half_lane) = u32x2{H::pack(x[0], x[1]), H::pack(x[2], x[3])};
        }
      lds_sync();
      // OCH lanes per staged row, 64 / OCH rows per access.
#pragma unroll
      for (int k = 0; k < 32 * OCH / 64; ++k) {
        const int rr = k * (64 / OCH) + lane / OCH;
        const u32x4 v = *(const u32x4*)(sp + rr * WTN + (rc ^ swz_o(rr)) * 8);
        const int row = wrow0 + i * 32 + rr;
        if (row < a.M && col < a.N) *(u32x4*)(C + (size_t)row * a.ld_out + col) = v;
      }
      lds_sync();
    }
  } else {
    // Paired read-back: 8 lanes per row, each with 4 columns of the first
    // block and the same 4 columns of the second; 8 rows per access.
    const int lr = lane >> 3;
    const int lc = 4 * (lane & 7);
    auto paired = [&](int i, int t, int t2) __attribute__((always_inline)) {
      const int col = wcol0 + t * 32 + lc;     // column of the first block's values
      const int col2 = wcol0 + t2 * 32 + lc;   // column of the second block's values
      // A rotation pair lies in one head, which is wholly rotated (Q, K) or
      // not (V), and wholly Q or not: both tests are wave-uniform.
      const bool rot = wcol0 + t * 32 < a.rope_cols;
      const bool isq = wcol0 + t * 32 < a.q_cols;
      // RoPE, rotate-half, over 64-column groups: column c < 32 of a group
      // pairs with c + 32, at frequency index 32 ((col % hd) / 64) + col % 32
      // (a 64-wide head is one group; a 128-wide head is packed as two).  The
      // (cos, sin) pairs of the lane's four rows are requested before any of
      // the piece's stores: the compiler cannot tell the table from the
      // output, and would otherwise hold each row's loads behind the previous
      // row's stores, one memory round trip per row.  Rows past M read the
      // last valid row and store nothing.
      float2 cs[4][4];
      if (rot) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = min(wrow0 + i * 32 + 8 * j + lr, a.M - 1);
          const float2* src = a.rope + (size_t)row * (a.hd >> 1) + 32 * ((col % a.hd) >> 6) + (col & 31);
#pragma unroll
          for (int e = 0; e < 4; ++e) cs[j][e] = src[e];
        }
      }
      lds_sync();
      uint16_t* C = (uint16_t*)tab.out_lo[g];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 8 * j + lr;
        const int row = wrow0 + i * 32 + r;
        f32x4 x1 = *(const f32x4*)(ep + r * EP_LD + lc);
        f32x4 x2 = *(const f32x4*)(ep + r * EP_LD + 32 + lc);
        if (row >= a.M || col >= a.N) continue;
        {
          if (rot) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float2 c = cs[j][e];
              const float y1 = x1[e] * c.x - x2[e] * c.y;
              const float y2 = x2[e] * c.x + x1[e] * c.y;
              x1[e] = y1;
              x2[e] = y2;
            }
          }
          if (isq) {   // Q: the attention scale
            x1 *= a.q_scale;
            x2 *= a.q_scale;
          }
          *(u32x2*)(C + (size_t)row * a.ld_out + col) = u32x2{H::pack(x1[0], x1[1]), H::pack(x1[2], x1[3])};
          *(u32x2*)(C + (size_t)row * a.ld_out + col2) = u32x2{H::pack(x2[0], x2[1]), H::pack(x2[2], x2[3])};
        }
      }
      lds_sync();
    };
    if constexpr (EPI == EPI_SWIGLU) {
      // The packed weight interleaves 32 gate and 32 up columns per 64-column
      // block, so the gate and up values of one output are element e of
      // blocks t and t + 1 in the same lane: SwiGLU runs in registers and only
      // its bf16 result, one 32 x 32 piece per block pair, goes through LDS.
      // Staged rows are 64 bytes whose 16-byte chunks are XOR-swizzled by
      // (row / 4) % 4, so the row-major read-back is bank-conflict free.
      constexpr int PIECES = MI * (NI / 2);
      static_assert(PIECES * 32 * 32 * 2 <= 32 * EP_LD * 4, "pieces fit the wave's region");
      uint16_t* sp = (uint16_t*)ep;
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int t = 0; t < NI; t += 2) {
          uint16_t* piece = sp + (i * (NI / 2) + t / 2) * 1024;
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) {
            float u[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float gv = acc[i][t][4 * e4 + q];
              u[q] = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * acc[i][t + 1][4 * e4 + q];
            }
            const int chunk = e4 ^ ((r32 >> 2) & 3);
            *(u32x2*)(piece + r32 * 32 + chunk * 8 + half_lane) =
                u32x2{H::pack(u[0], u[1]), H::pack(u[2], u[3])};
          }
        }
      lds_sync();
      // Read-back: 4 lanes per 64-byte row, 16 rows per access.
      const int rc = lane & 3;
      uint16_t* C = (uint16_t*)tab.out_lo[g];
      const int out_cols = a.N >> 1;
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int t = 0; t < NI; t += 2) {
          const uint16_t* piece = sp + (i * (NI / 2) + t / 2) * 1024;
          const int ocol = ((wcol0 + t * 32) >> 6) * 32 + rc * 8;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int rr = 16 * h + (lane >> 2);
            const u32x4 v = *(const u32x4*)(piece + rr * 32 + ((rc ^ ((rr >> 2) & 3)) * 8));
            const int row = wrow0 + i * 32 + rr;
            if (row < a.M && ocol < out_cols) *(u32x4*)(C + (size_t)row * a.ld_out + ocol) = v;
          }
        }
    } else {  // EPI_QKV_ROPE: the wave's columns start on a 64-column group
      // boundary (WTN is a multiple of 64), so block t pairs with t + 1.
      static_assert(NI % 2 == 0, "rotation groups must not straddle a wave's columns");
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int t = 0; t < NI; t += 2) {
          stage(acc[i][t], 0);
          stage(acc[i][t + 1], 1);
          paired(i, t, t + 1);
        }
    }
  }
}

// Weight slices take the non-temporal policy when K <= 2048: a cell's
// activations (M x K bf16, re-read by every column tile of the cell) are then
// about one XCD's L2, and streaming the weights past them saves ~1% on those
// GEMMs.  With longer K the activations exceed L2 anyway, and the reuse of a
// weight panel by the cell's row tiles matters more (the hint cost the
// K = 8192 projections 0.4-2%, and 2-4% at K = 4096).
template <int EPI, bool F16, int BM, int WTM, int WTN>
void launch_one(const GemmArgs& a, const GroupTable& tab, const NormAux& aux, hipStream_t stream) {
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN) * tab.G;
  constexpr int threads = (BM / WTM) * (BN / WTN) * 64;
  if (a.K <= 2048)
    hipLaunchKernelGGL((gemm_bf16_kernel<EPI, BM, WTM, WTN, true, F16>), dim3(tiles), dim3(threads), 0, stream, a, tab,
                       aux);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<EPI, BM, WTM, WTN, false, F16>), dim3(tiles), dim3(threads), 0, stream, a,
                       tab, aux);
}

// Tile shapes.  The operand bytes a tile pulls from L2 per MFMA fall as the
// tile grows, but a launch runs in rounds of one tile per CU, so the rows a
// tile leaves empty at a cell's end and a last round that is only partly
// filled cost as much as useful work.  Each launch takes the shape with the
// smallest estimated time, rounds x rows per tile / relative speed, the
// speeds measured on MI355X for 256-CU rounds:
//   288 x 256: twelve waves of 96 x 64 (3 x 2 blocks); a 1152-row cell is
//              exactly four tiles.                              speed 1.00
//   256 x 256: eight waves of 64 x 128 (2 x 4 blocks).           speed 0.95
//   192 x 256: eight waves of 96 x 64 (3 x 2 blocks).            speed 0.85
//   128 x 256: eight waves of 64 x 64.                          speed 0.72
// RoPE rotates within 64-column groups (128-wide heads are packed as two
// such groups), so every shape serves the QKV product.  Every shape uses the
// same K slicing and lane/k assignment, so a cell's result does not depend on
// the choice.
int num_cus() {
  static const int n = [] {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    return v;
  }();
  return n;
}

double tile_cost(const GemmArgs& a, int G, int bm, double speed) {
  const long tiles = (long)((a.M + bm - 1) / bm) * ((a.N + BN - 1) / BN) * G;
  const long rounds = (tiles + num_cus() - 1) / num_cus();
  return (double)rounds * bm / speed;
}

template <int EPI, bool F16>
void launch_epi(const GemmArgs& a, const GroupTable& tab, const NormAux& aux, hipStream_t stream) {
  const double c288 = tile_cost(a, tab.G, 288, 1.00);
  const double c256 = tile_cost(a, tab.G, 256, 0.95);
  const double c192 = tile_cost(a, tab.G, 192, 0.85);
  const double c128 = tile_cost(a, tab.G, 128, 0.72);
  if (c288 <= c256 && c288 <= c192 && c288 <= c128) {
    launch_one<EPI, F16, 288, 96, 64>(a, tab, aux, stream);
  } else if (c256 <= c192 && c256 <= c128) {
    launch_one<EPI, F16, 256, 64, 128>(a, tab, aux, stream);
  } else if (c192 <= c128) {
    launch_one<EPI, F16, 192, 96, 64>(a, tab, aux, stream);
  } else {
    launch_one<EPI, F16, 128, 64, 64>(a, tab, aux, stream);
  }
}

}  // namespace

hipError_t launch_gemm(int epilogue, const GemmArgs& a, const GroupTable& tab, hipStream_t stream,
                       const NormAux* aux_in) {
  if (tab.G == 0 || a.M == 0 || a.N == 0) return hipSuccess;
  const bool plain_store = epilogue == EPI_STORE_BF16 || epilogue == EPI_BIAS_BF16 ||
                           epilogue == EPI_BIAS_RELU_BF16;
  if (plain_store && a.N % 8 != 0) return hipErrorInvalidValue;   // whole 16-byte output chunks
  if (a.q_cols < 0 || a.q_cols % 32 != 0) return hipErrorInvalidValue;   // whole 32-column blocks
  if (epilogue == EPI_QKV_ROPE && (a.rope_cols < 0 || a.rope_cols % 64 != 0 || (a.hd != 64 && a.hd != 128)))
    return hipErrorInvalidValue;   // whole 64-column rotation groups
  if (a.a_split < 0 || a.a_split % 8 != 0 || (a.a_split > 0 && epilogue != EPI_QKV_ROPE))
    return hipErrorInvalidValue;   // whole 8-row loads on each side of the split
  const bool resid = epilogue == EPI_RESID_F32 || epilogue == EPI_RESID_BIAS_F32 || epilogue == EPI_RESID_NORM_F32;
  if (resid && a.N % 32 != 0) return hipErrorInvalidValue;   // whole 32-column blocks
  if (epilogue == EPI_RESID_NORM_F32 && (!aux_in || !a.aux_gamma || a.N % kChunk != 0))
    return hipErrorInvalidValue;
  if (epilogue == EPI_RESID_NORM_F32) {
    for (int g = 0; g < tab.G; ++g)      // every side output has a destination
      if (!aux_in->rows_lo[g] || !aux_in->rows_hi[g] || !aux_in->ss_lo[g] || !aux_in->ss_hi[g])
        return hipErrorInvalidValue;
  }
  static const NormAux none{};
  const NormAux& aux = aux_in ? *aux_in : none;
  if (a.f16) {
    // fp16 operands: the epilogues of the LLaMA-shaped cell and the plain store
    switch (epilogue) {
      case EPI_STORE_BF16: launch_epi<EPI_STORE_BF16, true>(a, tab, aux, stream); break;
      case EPI_QKV_ROPE: launch_epi<EPI_QKV_ROPE, true>(a, tab, aux, stream); break;
      case EPI_SWIGLU: launch_epi<EPI_SWIGLU, true>(a, tab, aux, stream); break;
      case EPI_RESID_F32: launch_epi<EPI_RESID_F32, true>(a, tab, aux, stream); break;
      case EPI_RESID_NORM_F32: launch_epi<EPI_RESID_NORM_F32, true>(a, tab, aux, stream); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  switch (epilogue) {
    case EPI_STORE_BF16: launch_epi<EPI_STORE_BF16, false>(a, tab, aux, stream); break;
    case EPI_QKV_ROPE: launch_epi<EPI_QKV_ROPE, false>(a, tab, aux, stream); break;
    case EPI_SWIGLU: launch_epi<EPI_SWIGLU, false>(a, tab, aux, stream); break;
    case EPI_RESID_F32: launch_epi<EPI_RESID_F32, false>(a, tab, aux, stream); break;
    case EPI_RESID_NORM_F32: launch_epi<EPI_RESID_NORM_F32, false>(a, tab, aux, stream); break;
    case EPI_BIAS_BF16: launch_epi<EPI_BIAS_BF16, false>(a, tab, aux, stream); break;
    case EPI_BIAS_RELU_BF16: launch_epi<EPI_BIAS_RELU_BF16, false>(a, tab, aux, stream); break;
    case EPI_RESID_BIAS_F32: launch_epi<EPI_RESID_BIAS_F32, false>(a, tab, aux, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rmt
