// Host runtime of librmt.so: the C ABI declared in include/rmt.h.
//
// The diagonal driver walks the anti-diagonals d = l + s of the
// (layer, segment) grid ("Diagonal Batching for Recurrent Memory
// Transformers", skill page: Implementation, the scheduler's enumeration;
// Architecture Overview, Diagonal Reorganization) and, for each diagonal,
// queues one grouped launch per stage of the cell over all of the diagonal's
// cells.  The per-cell group table (layer id and row pointers) travels in the
// kernel arguments, so no device memory depends on the number of segments.
//
// Buffers and hazards.  Two facts keep the grouped launches race-free:
//   * X(l, s) goes to a ping-pong pair: a cell on diagonal k reads slot l of
//     buffer (k+1) % 2 and writes slot l+1 of buffer k % 2.  Cell (l-1, s+1)
//     of the same diagonal therefore never overwrites the X(l-1, s) that
//     cell (l, s) is reading.  Slot 0 holds the segment's input rows.
//   * M(l, s) goes to one of two memory buffers by the parity of s: the one
//     the caller asked for (out->mem) when S-1-s is even, the workspace copy
//     otherwise.  A cell reads M(l, s-1) from one and writes M(l, s) to the
//     other, so the write-back never lands on rows another tile of the same
//     launch still reads as its residual, and M(., S-1) ends in out->mem
//     without a final copy.
// The LLaMA cell's RMSNorm inputs (16-bit copies y * gamma and chunk sums of
// y^2, written by whoever produces the rows) travel with their rows: X
// copies in slot l+1 of the X buffer being written, M copies in the memory
// buffer of M's parity, so the same two facts cover them.
// With B sequences (rmt_model_set_batch) every sequence has its own X
// ping-pong pair and memory buffers, and a diagonal's launches cover the
// cells of all B sequences (layer-major, sequence fastest, so cells of one
// layer sit next to each other and share weight panels in L2).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/rmt.h"
#include "kernels.h"

using namespace rmt;

// Activation workspace of rmt_forward_diagonal_static, for callers that cannot
// allocate device memory.  Each device the library runs on holds its own copy
// until the process ends; calls that overlap on one device share it.
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {

thread_local std::string g_last_error;

int32_t fail(int32_t code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

#define HIP_TRY(expr)                                                                   \
  do {                                                                                  \
    hipError_t e_ = (expr);                                                             \
    if (e_ != hipSuccess)                                                               \
      return fail(RMT_EHIP, "%s failed: %s", #expr, hipGetErrorString(e_));             \
  } while (0)

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace

struct rmt_model {
  rmt_config cfg{};
  hipStream_t stream = nullptr;
  rmt_weights src{};       // mathematical-layout weights, borrowed until they are packed
  // Caller-owned device buffers (rmt_model_bind); the library allocates none.
  void* wbuf = nullptr;    // packed weights, gains, RoPE table, flag
  size_t wbuf_bytes = 0;
  void* ws = nullptr;      // activation workspace, carved for the current batch
  size_t ws_bytes = 0;
  bool ws_ok = false;      // the bound workspace holds the current batch's pieces
  int batch = 1;           // sequences per forward call
  int n_last = 0;          // rows of the last segment: n, or fewer when T is not a multiple of n

  // packed weights (bf16, [L][N][K]) and gains (fp32)
  uint16_t* wqkv = nullptr;
  uint16_t* wo = nullptr;
  uint16_t* wgu = nullptr;
  uint16_t* wd = nullptr;
  float* g1 = nullptr;
  float* g2 = nullptr;
  // ENCODER: LayerNorm shifts and biases (fp32, [L][width])
  float* beta1 = nullptr;
  float* beta2 = nullptr;
  float* bqkv = nullptr;
  float* bo = nullptr;
  float* b1 = nullptr;
  float* b2 = nullptr;
  float* w32 = nullptr;    // LINEAR_GELU: [L][d][d]
  float* b32 = nullptr;    // LINEAR_GELU: [L][d]
  const uint16_t* embed = nullptr;  // borrowed
  float2* rope = nullptr;  // [R][hd/2] (cos, sin)

  // workspace: per-launch buffers for up to C = min(kMaxGroups, B*L) cells,
  // and per-sequence X ping-pong and memory buffers
  uint16_t* abuf = nullptr;  // normalised rows, bf16 [C*R][d]
  uint16_t* qkv = nullptr;   // [C*R][Nqkv]
  uint16_t* att = nullptr;   // [C*R][Hq*hd]
  float* hbuf = nullptr;     // [C*R][d]
  float* h2buf = nullptr;    // [C*R][d] (post-norm ENCODER: H after LayerNorm 1)
  uint16_t* ubuf = nullptr;  // [C*R][F]
  float* xbuf[2] = {nullptr, nullptr};  // [B][L][n][d] each
  float* memw = nullptr;     // [B][L][m][d]
  // LLAMA: RMSNorm inputs prepared by the producers of the rows (16-bit
  // copies y * gamma and 64-column chunk sums of y^2): X slots (parallel to
  // xbuf), memory rows (parallel to the two memory buffers, same parity), and
  // the per-launch H rows; rinv holds the launch's 1/rms per row.
  // X slots of the 16-bit copies: slot l holds X(l-1, .); slot L takes the
  // last layer's copies, which no cell reads
  uint16_t* xb16[2] = {nullptr, nullptr};  // [B][L+1][n][d]
  float* xss[2] = {nullptr, nullptr};      // [B][L+1] slots of [d/64][n] (chunk-major)
  uint16_t* mb16[2] = {nullptr, nullptr};  // [B][L][m][d]; [0] pairs with out->mem, [1] with memw
  float* mss[2] = {nullptr, nullptr};      // [B][L] slots of [d/64][m]
  float* hss = nullptr;      // [C] cells of [d/64][R]
  float* rinv = nullptr;     // [C*R]
  int32_t* flag = nullptr;   // bad-token flag

  // timing
  bool timing = false;
  std::vector<hipEvent_t> events;   // pool
  size_t ev_used = 0;
  std::vector<int> ev_stage;        // stage of the launch that ends at event i (-1: start marker)
  std::vector<double> ev_flops, ev_bytes;
  std::vector<int> ev_groups;       // cells covered by that launch (0: not a per-diagonal launch)
  int cur_groups = 0;               // cells of the launches being queued
};

namespace {

int nqkv(const rmt_config& c) { return (c.n_heads + 2 * c.n_kv_heads) * c.head_dim; }

bool has_attention(const rmt_config& c) { return c.cell == RMT_CELL_LLAMA || c.cell == RMT_CELL_ENCODER; }

bool head_ratio_ok(int Hq, int Hkv) {
  if (Hkv < 1 || Hq < 1 || Hq % Hkv != 0) return false;
  const int rep = Hq / Hkv;
  return rep == 1 || rep == 2 || rep % 4 == 0;
}

int32_t validate_config(const rmt_config* c) {
  if (!c) return fail(RMT_EINVAL, "config is NULL");
  if (c->L < 1 || c->S < 1 || c->n < 1 || c->m < 1 || c->d < 1)
    return fail(RMT_EINVAL, "L, S, n, m, d must be >= 1 (got %d, %d, %d, %d, %d)", c->L, c->S, c->n,
                c->m, c->d);
  const int64_t R = (int64_t)c->n + c->m;
  if (c->cell == RMT_CELL_LINEAR_GELU) {
    if (c->dtype != RMT_F32) return fail(RMT_EUNSUPPORTED, "LINEAR_GELU cells run in fp32 only");
    if ((int64_t)c->L * R * c->d > INT32_MAX) return fail(RMT_EINVAL, "sizes overflow int32");
    return RMT_OK;
  }
  if (c->cell != RMT_CELL_NORM_SWIGLU && c->cell != RMT_CELL_LLAMA && c->cell != RMT_CELL_ENCODER)
    return fail(RMT_EINVAL, "unknown cell kind %d", c->cell);
  if (c->dtype != RMT_BF16 && !(c->dtype == RMT_F16 && c->cell == RMT_CELL_LLAMA))
    return fail(RMT_EUNSUPPORTED, "this cell kind runs in bf16 only (fp16 operands: LLAMA cells)");
  if (c->d % 64 != 0) return fail(RMT_EUNSUPPORTED, "d must be a multiple of 64 (got %d)", c->d);
  if (c->ffn < 1 || c->ffn % 32 != 0)
    return fail(RMT_EUNSUPPORTED, "ffn must be a positive multiple of 32 (got %d)", c->ffn);
  if (!(c->eps >= 0.f)) return fail(RMT_EINVAL, "eps must be >= 0");
  int64_t widest = std::max<int64_t>(c->d, c->ffn);
  if (has_attention(*c)) {
    if (c->n_heads < 1 || c->n_kv_heads < 1 || c->n_heads % c->n_kv_heads != 0)
      return fail(RMT_EINVAL, "n_heads must be a positive multiple of n_kv_heads");
    if (c->cell == RMT_CELL_ENCODER && c->n_kv_heads != c->n_heads)
      return fail(RMT_EUNSUPPORTED, "ENCODER cells have one KV head per query head");
    if (!head_ratio_ok(c->n_heads, c->n_kv_heads))
      return fail(RMT_EUNSUPPORTED, "n_heads / n_kv_heads must be 1, 2 or a multiple of 4");
    if (c->head_dim != 64 && c->head_dim != 128)
      return fail(RMT_EUNSUPPORTED, "head_dim must be 64 or 128 (got %d)", c->head_dim);
    if (c->n_heads * c->head_dim != c->d)
      return fail(RMT_EUNSUPPORTED, "n_heads * head_dim must equal d");
    widest = std::max<int64_t>(widest, nqkv(*c));
  }
  if (c->post_norm != 0 && (c->cell != RMT_CELL_ENCODER || c->post_norm != 1))
    return fail(RMT_EINVAL, "post_norm is 0 or 1, and 1 only for ENCODER cells");
  if (c->cell == RMT_CELL_LLAMA) {
    if (c->vocab < 1) return fail(RMT_EINVAL, "vocab must be >= 1");
    if (c->m % 8 != 0) return fail(RMT_EUNSUPPORTED, "LLAMA cells need m a multiple of 8 (got %d)", c->m);
    if (!(c->rope_theta > 0.f)) return fail(RMT_EINVAL, "rope_theta must be > 0");
  }
  if ((int64_t)c->L * R * 2 * widest > INT32_MAX) return fail(RMT_EINVAL, "sizes overflow int32");
  if ((int64_t)c->S * c->n * c->d > ((int64_t)1 << 40)) return fail(RMT_EINVAL, "sequence too long");
  return RMT_OK;
}

// ---------------------------------------------------------------------------
// Timing helpers
// ---------------------------------------------------------------------------

int32_t mark(rmt_model* M, int stage, double flops, double bytes) {
  if (!M->timing) return RMT_OK;
  if (M->ev_used == M->events.size()) {
    hipEvent_t e;
    HIP_TRY(hipEventCreate(&e));
    M->events.push_back(e);
  }
  HIP_TRY(hipEventRecord(M->events[M->ev_used], M->stream));
  M->ev_used++;
  M->ev_stage.push_back(stage);
  M->ev_flops.push_back(flops);
  M->ev_bytes.push_back(bytes);
  M->ev_groups.push_back(M->cur_groups);
  return RMT_OK;
}

#define LAUNCH(expr)                                                                     \
  do {                                                                                   \
    hipError_t e_ = (expr);                                                              \
    if (e_ != hipSuccess) return fail(RMT_EHIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

#define MARK(stage, fl, by)                          \
  do {                                               \
    int32_t r_ = mark(M, (stage), (fl), (by));       \
    if (r_ != RMT_OK) return r_;                     \
  } while (0)

struct Cell {
  int l, s, b;   // layer, segment, sequence
};

// Queue every stage of the cells in `cells` (all on anti-diagonal k, at most
// kMaxGroups of them).
int32_t run_cells(rmt_model* M, const Cell* cells, int G, const void* tokens, const rmt_output* out) {
  const rmt_config& c = M->cfg;
  const int L = c.L, S = c.S, n = c.n, m = c.m, d = c.d;
  // Every cell of one launch has the same number of segment rows: n, or
  // n_last for the cells of a short last segment (rmt_forward_diagonal
  // launches those on their own).
  const int ns = cells[0].s == S - 1 ? M->n_last : n;
  const int R = ns + m;
  const int k = cells[0].l + cells[0].s;
  const size_t T = (size_t)(S - 1) * n + M->n_last;   // tokens per sequence
  float* xr = M->xbuf[(k + 1) & 1];
  float* xw = M->xbuf[k & 1];
  // slot l of sequence b's X buffer; sequence b's memory buffer for segment s
  auto slot = [&](float* buf, int b, int l) { return buf + ((size_t)b * L + l) * n * d; };
  auto mem_buf = [&](int b, int s) {
    return (((S - 1 - s) % 2 == 0) ? out->mem : M->memw) + (size_t)b * L * m * d;
  };
  const double G_ = G;
  M->cur_groups = G;

  // Cell inputs [M(l, s-1); X(l-1, s)] and outputs X(l, s), M(l, s).
  const void* in_lo[kMaxGroups];
  const void* in_hi[kMaxGroups];
  void* x_out[kMaxGroups];
  void* m_out[kMaxGroups];
  for (int g = 0; g < G; ++g) {
    const int l = cells[g].l, s = cells[g].s, b = cells[g].b;
    const size_t tok0 = (size_t)b * T + (size_t)s * n;   // first token of segment s of sequence b
    in_lo[g] = mem_buf(b, s - 1) + (size_t)l * m * d;
    if (l == 0 && c.cell == RMT_CELL_LINEAR_GELU)
      in_hi[g] = (const float*)tokens + tok0 * d;   // fp32 input rows, read in place
    else
      in_hi[g] = slot(xr, b, l);
    x_out[g] = (l == L - 1) ? (void*)(out->hidden + tok0 * d) : (void*)slot(xw, b, l + 1);
    m_out[g] = mem_buf(b, s) + (size_t)l * m * d;
    if (l == 0 && c.cell != RMT_CELL_LINEAR_GELU) {
      // X(-1, s): this segment's input rows, into slot 0 of the read buffer.
      if (c.cell == RMT_CELL_LLAMA) {
        // with the RMSNorm-1 inputs of layer 0: 16-bit copy and chunk sums
        const size_t nc = d / kChunk;
        LAUNCH(launch_gather_tokens(ns, d, (const int32_t*)tokens + tok0, c.vocab, M->embed,
                                    slot(xr, b, 0), M->flag, M->stream, M->g1,
                                    M->xb16[(k + 1) & 1] + (size_t)b * (L + 1) * n * d,
                                    M->xss[(k + 1) & 1] + (size_t)b * (L + 1) * n * nc, n, c.dtype == RMT_F16));
        MARK(RMT_STAGE_GATHER, 0.0, (double)ns * (4 + (size_t)d * 8 + nc * 4));
      } else {
        LAUNCH(launch_copy_rows_bf16(ns, d, (const uint16_t*)tokens + tok0 * d, slot(xr, b, 0),
                                     M->stream));
        MARK(RMT_STAGE_GATHER, 0.0, (double)ns * d * 6);
      }
    }
  }

  GroupTable tab;
  std::memset(&tab, 0, sizeof(tab));
  tab.G = G;
  for (int g = 0; g < G; ++g) tab.layer[g] = cells[g].l;
  auto set_io = [&](const void* const* lo, const void* const* hi, void* const* olo, void* const* ohi) {
    for (int g = 0; g < G; ++g) {
      tab.in_lo[g] = lo ? lo[g] : nullptr;
      tab.in_hi[g] = hi ? hi[g] : nullptr;
      tab.out_lo[g] = olo ? olo[g] : nullptr;
      tab.out_hi[g] = ohi ? ohi[g] : nullptr;
    }
  };
  const double rows = G_ * R;

  if (c.cell == RMT_CELL_LINEAR_GELU) {
    set_io(in_lo, in_hi, x_out, m_out);
    LAUNCH(launch_linear_gelu_f32(G, R, d, m, ns, tab, M->w32, M->b32, M->stream));
    MARK(RMT_STAGE_LINEAR, 2.0 * rows * d * d, rows * d * 8 + G_ * d * (d + 1) * 4);
    return RMT_OK;
  }

  const int F = c.ffn;
  const void* packed_lo[kMaxGroups];
  void* packed_out[kMaxGroups];
  GemmArgs ga;
  std::memset(&ga, 0, sizeof(ga));

  const bool f16 = c.dtype == RMT_F16;   // LLAMA cells only: every 16-bit operand in fp16
  ga.f16 = f16;
  NormAux ax;
  std::memset(&ax, 0, sizeof(ax));
  const size_t nc = d / kChunk;
  // memory-buffer parity of segment s (the buffer mem_buf picks), for the
  // memory rows' 16-bit copies and chunk sums
  auto mpar = [&](int s) { return ((S - 1 - s) % 2 == 0) ? 0 : 1; };
  if (c.cell == RMT_CELL_LLAMA) {
    const int hd = c.head_dim, Hq = c.n_heads, Hkv = c.n_kv_heads, NQ = nqkv(c);
    const int pr = (k + 1) & 1;    // X read parity
    // RMSNorm 1 of [M(l, s-1); X(l-1, s)]: 1/rms per row from the chunk sums
    // that the rows' producers wrote (down projections, gather, memory prep)
    for (int g = 0; g < G; ++g) {
      const int l = cells[g].l, s = cells[g].s, b = cells[g].b;
      ax.ss_lo[g] = M->mss[mpar(s - 1)] + ((size_t)b * L + l) * m * nc;
      ax.ss_hi[g] = M->xss[pr] + ((size_t)b * (L + 1) + l) * n * nc;
    }
    ax.ss_ld_lo = m;
    ax.ss_ld_hi = n;
    LAUNCH(launch_row_rinv(G, R, d, m, ax, c.eps, M->rinv, M->stream));
    MARK(RMT_STAGE_NORM1, 0.0, rows * (nc * 4 + 4));
    // QKV projection of the rows' 16-bit copies y * g1 (memory rows, then
    // segment rows), scaled by 1/rms per row, + RoPE on Q and K
    for (int g = 0; g < G; ++g) {
      const int l = cells[g].l, s = cells[g].s, b = cells[g].b;
      tab.in_lo[g] = M->mb16[mpar(s - 1)] + ((size_t)b * L + l) * m * d;
      tab.in_hi[g] = M->xb16[pr] + ((size_t)b * (L + 1) + l) * n * d;
      tab.out_lo[g] = M->qkv + (size_t)g * R * NQ;
      tab.out_hi[g] = nullptr;
    }
    ga.A = nullptr; ga.B = M->wqkv; ga.M = R; ga.N = NQ; ga.K = d;
    ga.split_in = R; ga.split_out = R; ga.ld_res = 0; ga.ld_out = NQ;
    ga.rope = M->rope; ga.rope_cols = (Hq + Hkv) * hd; ga.hd = hd;
    ga.q_cols = Hq * hd; ga.q_scale = attention_scale_log2(hd);   // Q leaves with the softmax scale
    ga.a_split = m; ga.row_scale = M->rinv;
    LAUNCH(launch_gemm(EPI_QKV_ROPE, ga, tab, M->stream));
    ga.q_cols = 0; ga.a_split = 0; ga.row_scale = nullptr;
    MARK(RMT_STAGE_QKV, 2.0 * rows * d * NQ, rows * d * 2 + G_ * NQ * d * 2 + rows * NQ * 2 + rows * 4);
    // causal GQA attention inside each cell
    LAUNCH(launch_attention(M->qkv, M->att, G, R, Hq, Hkv, hd, true, true, M->stream, f16));
    MARK(RMT_STAGE_ATTN, 2.0 * G_ * Hq * hd * (double)R * (R + 1), rows * NQ * 2 + rows * Hq * hd * 2);
    // O projection + residual A -> H (fp32), and H's RMSNorm-2 inputs: the
    // 16-bit copy H * g2 (the gate/up operand) and its chunk sums
    for (int g = 0; g < G; ++g) packed_out[g] = M->hbuf + (size_t)g * R * d;
    std::memset(&ax, 0, sizeof(ax));
    for (int g = 0; g < G; ++g) {
      ax.rows_lo[g] = ax.rows_hi[g] = M->abuf + (size_t)g * R * d;   // every row is "lo" (split R)
      ax.ss_lo[g] = ax.ss_hi[g] = M->hss + (size_t)g * R * nc;
      ax.layer_lo[g] = ax.layer_hi[g] = cells[g].l;
    }
    ax.ss_ld_lo = ax.ss_ld_hi = R;
    set_io(in_lo, in_hi, packed_out, nullptr);
    ga.A = M->att; ga.B = M->wo; ga.M = R; ga.N = d; ga.K = Hq * hd;
    ga.split_in = m; ga.split_out = R; ga.ld_res = d; ga.ld_out = d;
    ga.aux_gamma = M->g2;
    LAUNCH(launch_gemm(EPI_RESID_NORM_F32, ga, tab, M->stream, &ax));
    ga.aux_gamma = nullptr;
    MARK(RMT_STAGE_OPROJ, 2.0 * rows * Hq * hd * d,
         rows * Hq * hd * 2 + G_ * d * Hq * hd * 2 + rows * d * 10 + rows * nc * 4);
    // RMSNorm 2: 1/rms per row of H
    LAUNCH(launch_row_rinv(G, R, d, R, ax, c.eps, M->rinv, M->stream));
    MARK(RMT_STAGE_NORM2, 0.0, rows * (nc * 4 + 4));
  } else if (c.cell == RMT_CELL_ENCODER && c.post_norm) {
    const int hd = c.head_dim, H = c.n_heads, NQ = nqkv(c);
    // A = [M(l, s-1); X(l-1, s)] as bf16 (the attention sees A itself)
    set_io(in_lo, in_hi, nullptr, nullptr);
    LAUNCH(launch_cast_rows(G, R, d, m, tab, M->abuf, M->stream));
    MARK(RMT_STAGE_NORM1, 0.0, rows * d * 6);
    // Q, K, V projection + bias
    for (int g = 0; g < G; ++g) packed_out[g] = M->qkv + (size_t)g * R * NQ;
    set_io(nullptr, nullptr, packed_out, nullptr);
    ga.A = M->abuf; ga.B = M->wqkv; ga.M = R; ga.N = NQ; ga.K = d;
    ga.split_in = R; ga.split_out = R; ga.ld_res = 0; ga.ld_out = NQ; ga.bias = M->bqkv;
    ga.q_cols = H * hd; ga.q_scale = attention_scale_log2(hd);    // Q leaves with the softmax scale
    LAUNCH(launch_gemm(EPI_BIAS_BF16, ga, tab, M->stream));
    ga.q_cols = 0;
    MARK(RMT_STAGE_QKV, 2.0 * rows * d * NQ, rows * d * 2 + G_ * NQ * d * 2 + rows * NQ * 2);
    LAUNCH(launch_attention(M->qkv, M->att, G, R, H, H, hd, false, true, M->stream));
    MARK(RMT_STAGE_ATTN, 4.0 * G_ * H * hd * (double)R * R, rows * NQ * 2 + rows * H * hd * 2);
    // O projection + bias + residual A -> hbuf (before LayerNorm 1)
    for (int g = 0; g < G; ++g) packed_out[g] = M->hbuf + (size_t)g * R * d;
    set_io(in_lo, in_hi, packed_out, nullptr);
    ga.A = M->att; ga.B = M->wo; ga.M = R; ga.N = d; ga.K = H * hd;
    ga.split_in = m; ga.split_out = R; ga.ld_res = d; ga.ld_out = d; ga.bias = M->bo;
    LAUNCH(launch_gemm(EPI_RESID_BIAS_F32, ga, tab, M->stream));
    MARK(RMT_STAGE_OPROJ, 2.0 * rows * H * hd * d, rows * H * hd * 2 + G_ * d * H * hd * 2 + rows * d * 8);
    // H = LayerNorm 1 -> h2buf (fp32, the residual stream) and abuf (bf16, the W1 operand)
    const void* hb_lo[kMaxGroups];
    void* h2_out[kMaxGroups];
    for (int g = 0; g < G; ++g) {
      hb_lo[g] = M->hbuf + (size_t)g * R * d;
      h2_out[g] = M->h2buf + (size_t)g * R * d;
    }
    set_io(hb_lo, hb_lo, h2_out, h2_out);
    LAUNCH(launch_layernorm_f32(G, R, d, R, R, tab, M->g1, M->beta1, c.eps, M->abuf, M->stream));
    MARK(RMT_STAGE_NORM2, 0.0, rows * d * 10);
    // W1 + bias + ReLU -> U
    for (int g = 0; g < G; ++g) packed_out[g] = M->ubuf + (size_t)g * R * F;
    set_io(nullptr, nullptr, packed_out, nullptr);
    ga.A = M->abuf; ga.B = M->wgu; ga.M = R; ga.N = F; ga.K = d;
    ga.split_in = R; ga.split_out = R; ga.ld_res = 0; ga.ld_out = F; ga.bias = M->b1;
    LAUNCH(launch_gemm(EPI_BIAS_RELU_BF16, ga, tab, M->stream));
    MARK(RMT_STAGE_GATEUP, 2.0 * rows * d * F, rows * d * 2 + G_ * F * d * 2 + rows * F * 2);
    // W2 + bias + residual H -> hbuf (before LayerNorm 2)
    const void* h2_lo[kMaxGroups];
    void* hb_out[kMaxGroups];
    for (int g = 0; g < G; ++g) {
      h2_lo[g] = M->h2buf + (size_t)g * R * d;
      hb_out[g] = M->hbuf + (size_t)g * R * d;
    }
    set_io(h2_lo, h2_lo, hb_out, hb_out);
    ga.A = M->ubuf; ga.B = M->wd; ga.M = R; ga.N = d; ga.K = F;
    ga.split_in = R; ga.split_out = R; ga.ld_res = d; ga.ld_out = d; ga.bias = M->b2;
    LAUNCH(launch_gemm(EPI_RESID_BIAS_F32, ga, tab, M->stream));
    MARK(RMT_STAGE_DOWN, 2.0 * rows * F * d, rows * F * 2 + G_ * d * F * 2 + rows * d * 8);
    // Y = LayerNorm 2; rows [0, n) -> X(l, s), rows [n, R) -> M(l, s)
    set_io(hb_lo, hb_lo, x_out, m_out);
    LAUNCH(launch_layernorm_f32(G, R, d, R, ns, tab, M->g2, M->beta2, c.eps, nullptr, M->stream));
    MARK(RMT_STAGE_NORM2, 0.0, rows * d * 8);
    return RMT_OK;
  } else if (c.cell == RMT_CELL_ENCODER) {
    const int hd = c.head_dim, H = c.n_heads, NQ = nqkv(c);
    // LayerNorm 1 of [M(l, s-1); X(l-1, s)]
    set_io(in_lo, in_hi, nullptr, nullptr);
    LAUNCH(launch_layernorm(G, R, d, m, tab, M->g1, M->beta1, c.eps, M->abuf, M->stream));
    MARK(RMT_STAGE_NORM1, 0.0, rows * d * 6);
    // Q, K, V projection + bias
    for (int g = 0; g < G; ++g) packed_out[g] = M->qkv + (size_t)g * R * NQ;
    set_io(nullptr, nullptr, packed_out, nullptr);
    ga.A = M->abuf; ga.B = M->wqkv; ga.M = R; ga.N = NQ; ga.K = d;
    ga.split_in = R; ga.split_out = R; ga.ld_res = 0; ga.ld_out = NQ; ga.bias = M->bqkv;
    ga.q_cols = H * hd; ga.q_scale = attention_scale_log2(hd);    // Q leaves with the softmax scale
    LAUNCH(launch_gemm(EPI_BIAS_BF16, ga, tab, M->stream));
    ga.q_cols = 0;
    MARK(RMT_STAGE_QKV, 2.0 * rows * d * NQ, rows * d * 2 + G_ * NQ * d * 2 + rows * NQ * 2);
    // unmasked multi-head attention inside each cell
    LAUNCH(launch_attention(M->qkv, M->att, G, R, H, H, hd, false, true, M->stream));
    MARK(RMT_STAGE_ATTN, 4.0 * G_ * H * hd * (double)R * R, rows * NQ * 2 + rows * H * hd * 2);
    // O projection + bias + residual A -> H
    for (int g = 0; g < G; ++g) packed_out[g] = M->hbuf + (size_t)g * R * d;
    set_io(in_lo, in_hi, packed_out, nullptr);
    ga.A = M->att; ga.B = M->wo; ga.M = R; ga.N = d; ga.K = H * hd;
    ga.split_in = m; ga.split_out = R; ga.ld_res = d; ga.ld_out = d; ga.bias = M->bo;
    LAUNCH(launch_gemm(EPI_RESID_BIAS_F32, ga, tab, M->stream));
    MARK(RMT_STAGE_OPROJ, 2.0 * rows * H * hd * d, rows * H * hd * 2 + G_ * d * H * hd * 2 + rows * d * 8);
    // LayerNorm 2 of H
    for (int g = 0; g < G; ++g) packed_lo[g] = M->hbuf + (size_t)g * R * d;
    set_io(packed_lo, packed_lo, nullptr, nullptr);
    LAUNCH(launch_layernorm(G, R, d, R, tab, M->g2, M->beta2, c.eps, M->abuf, M->stream));
    MARK(RMT_STAGE_NORM2, 0.0, rows * d * 6);
    // W1 + bias + ReLU -> U
    for (int g = 0; g < G; ++g) packed_out[g] = M->ubuf + (size_t)g * R * F;
    set_io(nullptr, nullptr, packed_out, nullptr);
    ga.A = M->abuf; ga.B = M->wgu; ga.M = R; ga.N = F; ga.K = d;
    ga.split_in = R; ga.split_out = R; ga.ld_res = 0; ga.ld_out = F; ga.bias = M->b1;
    LAUNCH(launch_gemm(EPI_BIAS_RELU_BF16, ga, tab, M->stream));
    MARK(RMT_STAGE_GATEUP, 2.0 * rows * d * F, rows * d * 2 + G_ * F * d * 2 + rows * F * 2);
    // W2 + bias + residual H; rows [0, n) -> X(l, s), rows [n, R) -> M(l, s)
    set_io(packed_lo, packed_lo, x_out, m_out);
    ga.A = M->ubuf; ga.B = M->wd; ga.M = R; ga.N = d; ga.K = F;
    ga.split_in = R; ga.split_out = ns; ga.ld_res = d; ga.ld_out = d; ga.bias = M->b2;
    LAUNCH(launch_gemm(EPI_RESID_BIAS_F32, ga, tab, M->stream));
    MARK(RMT_STAGE_DOWN, 2.0 * rows * F * d, rows * F * 2 + G_ * d * F * 2 + rows * d * 8);
    return RMT_OK;
  } else {
    // NORM_SWIGLU: RMSNorm of [M(l, s-1); X(l-1, s)]
    set_io(in_lo, in_hi, nullptr, nullptr);
    LAUNCH(launch_rmsnorm(G, R, d, m, tab, M->g2, c.eps, M->abuf, M->stream));
    MARK(RMT_STAGE_NORM2, 0.0, rows * d * 6);
  }

  // gate/up projection + SwiGLU -> U
  for (int g = 0; g < G; ++g) packed_out[g] = M->ubuf + (size_t)g * R * F;
  set_io(nullptr, nullptr, packed_out, nullptr);
  ga.A = M->abuf; ga.B = M->wgu; ga.M = R; ga.N = 2 * F; ga.K = d;
  ga.split_in = R; ga.split_out = R; ga.ld_res = 0; ga.ld_out = F;
  // LLAMA: abuf holds H * g2, and the rows take their 1/rms here
  ga.row_scale = c.cell == RMT_CELL_LLAMA ? M->rinv : nullptr;
  LAUNCH(launch_gemm(EPI_SWIGLU, ga, tab, M->stream));
  ga.row_scale = nullptr;
  MARK(RMT_STAGE_GATEUP, 2.0 * rows * d * 2 * F,
       rows * d * 2 + G_ * 2 * F * d * 2 + rows * F * 2 + (c.cell == RMT_CELL_LLAMA ? rows * 4 : 0));

  // down projection + residual; rows [0, n) -> X(l, s), rows [n, R) -> M(l, s)
  double aux_bytes = 0.0;
  if (c.cell == RMT_CELL_LLAMA) {
    for (int g = 0; g < G; ++g) packed_lo[g] = M->hbuf + (size_t)g * R * d;
    set_io(packed_lo, packed_lo, x_out, m_out);
    ga.split_in = R;
    // and the RMSNorm-1 inputs of the rows' next cells: X(l, s) for (l+1, s)
    // (gain g1[l+1]; none after the last layer), M(l, s) for (l, s+1) (gain
    // g1[l]; none after the last segment)
    std::memset(&ax, 0, sizeof(ax));
    const int pw = k & 1;
    for (int g = 0; g < G; ++g) {
      const int l = cells[g].l, s = cells[g].s, b = cells[g].b;
      // slot l+1 (slot L, a discard area, after the last layer)
      ax.rows_lo[g] = M->xb16[pw] + ((size_t)b * (L + 1) + l + 1) * n * d;
      ax.ss_lo[g] = M->xss[pw] + ((size_t)b * (L + 1) + l + 1) * n * nc;
      // after the last segment these copies are not read (the next forward
      // call prepares its own from the memory it is given)
      ax.rows_hi[g] = M->mb16[mpar(s)] + ((size_t)b * L + l) * m * d;
      ax.ss_hi[g] = M->mss[mpar(s)] + ((size_t)b * L + l) * m * nc;
      ax.layer_lo[g] = std::min(l + 1, L - 1);
      ax.layer_hi[g] = l;
    }
    ax.ss_ld_lo = n;
    ax.ss_ld_hi = m;
    aux_bytes = rows * ((double)d * 2 + nc * 4);
    ga.aux_gamma = M->g1;
  } else {
    set_io(in_lo, in_hi, x_out, m_out);
    ga.split_in = m;
  }
  ga.A = M->ubuf; ga.B = M->wd; ga.M = R; ga.N = d; ga.K = F;
  ga.split_out = ns; ga.ld_res = d; ga.ld_out = d;
  LAUNCH(launch_gemm(c.cell == RMT_CELL_LLAMA ? EPI_RESID_NORM_F32 : EPI_RESID_F32, ga, tab, M->stream, &ax));
  ga.aux_gamma = nullptr;
  MARK(RMT_STAGE_DOWN, 2.0 * rows * F * d, rows * F * 2 + G_ * d * F * 2 + rows * d * 8 + aux_bytes);
  return RMT_OK;
}

struct Piece {
  void** ptr;
  size_t bytes;
};

// Lay the pieces out one after another from `base` at 256-byte boundaries
// (base == nullptr: size only).  Returns the total size.
size_t carve(const std::vector<Piece>& pieces, void* base) {
  size_t off = 0;
  for (const auto& p : pieces) {
    off = align_up(off, 256);
    if (base) *p.ptr = (char*)base + off;
    off += p.bytes;
  }
  return align_up(off, 256);
}

// The packed weights and tables of the model's config: independent of S and B.
std::vector<Piece> weight_pieces(rmt_model* M) {
  const rmt_config& c = M->cfg;
  const size_t L = c.L, d = c.d, R = (size_t)c.n + c.m, F = c.ffn;
  const size_t NQ = has_attention(c) ? (size_t)nqkv(c) : 0;
  const size_t HQD = has_attention(c) ? (size_t)c.n_heads * c.head_dim : 0;
  std::vector<Piece> pieces;
  if (c.cell == RMT_CELL_LINEAR_GELU) {
    pieces.push_back({(void**)&M->w32, L * d * d * 4});
    pieces.push_back({(void**)&M->b32, L * d * 4});
  } else if (c.cell == RMT_CELL_ENCODER) {
    // W1 packed [L][F][d] in the `wgu` slot, W2 packed [L][d][F] in `wd`
    pieces.push_back({(void**)&M->wgu, L * F * d * 2});
    pieces.push_back({(void**)&M->wd, L * d * F * 2});
    pieces.push_back({(void**)&M->wqkv, L * NQ * d * 2});
    pieces.push_back({(void**)&M->wo, L * d * HQD * 2});
    pieces.push_back({(void**)&M->g1, L * d * 4});
    pieces.push_back({(void**)&M->beta1, L * d * 4});
    pieces.push_back({(void**)&M->g2, L * d * 4});
    pieces.push_back({(void**)&M->beta2, L * d * 4});
    pieces.push_back({(void**)&M->bqkv, L * NQ * 4});
    pieces.push_back({(void**)&M->bo, L * d * 4});
    pieces.push_back({(void**)&M->b1, L * F * 4});
    pieces.push_back({(void**)&M->b2, L * d * 4});
  } else {
    pieces.push_back({(void**)&M->wgu, L * 2 * F * d * 2});
    pieces.push_back({(void**)&M->wd, L * d * F * 2});
    pieces.push_back({(void**)&M->g2, L * d * 4});
    if (c.cell == RMT_CELL_LLAMA) {
      pieces.push_back({(void**)&M->wqkv, L * NQ * d * 2});
      pieces.push_back({(void**)&M->wo, L * d * HQD * 2});
      pieces.push_back({(void**)&M->g1, L * d * 4});
      pieces.push_back({(void**)&M->rope, R * (c.head_dim / 2) * sizeof(float2)});
    }
  }
  pieces.push_back({(void**)&M->flag, 256});
  return pieces;
}

// The activation workspace for B sequences: per-launch buffers for up to
// min(kMaxGroups, B*L) cells, and per-sequence X ping-pong and memory
// buffers.  Independent of S.
std::vector<Piece> workspace_pieces(rmt_model* M, int B) {
  const rmt_config& c = M->cfg;
  const size_t L = c.L, n = c.n, m = c.m, d = c.d, R = n + m, F = c.ffn;
  const size_t cells = std::min<size_t>(kMaxGroups, (size_t)B * L);
  const size_t rows = cells * R;
  std::vector<Piece> pieces;
  if (c.cell != RMT_CELL_LINEAR_GELU) {
    pieces.push_back({(void**)&M->abuf, rows * d * 2});
    pieces.push_back({(void**)&M->ubuf, rows * F * 2});
    if (has_attention(c)) {
      pieces.push_back({(void**)&M->qkv, rows * nqkv(c) * 2});
      pieces.push_back({(void**)&M->att, rows * (size_t)c.n_heads * c.head_dim * 2});
      pieces.push_back({(void**)&M->hbuf, rows * d * 4});
      if (c.post_norm) pieces.push_back({(void**)&M->h2buf, rows * d * 4});
    }
  }
  pieces.push_back({(void**)&M->xbuf[0], (size_t)B * L * n * d * 4});
  pieces.push_back({(void**)&M->xbuf[1], (size_t)B * L * n * d * 4});
  pieces.push_back({(void**)&M->memw, (size_t)B * L * m * d * 4});
  if (c.cell == RMT_CELL_LLAMA) {
    const size_t nc = d / kChunk;
    for (int p = 0; p < 2; ++p) {
      pieces.push_back({(void**)&M->xb16[p], (size_t)B * (L + 1) * n * d * 2});
      pieces.push_back({(void**)&M->xss[p], (size_t)B * (L + 1) * n * nc * 4});
      pieces.push_back({(void**)&M->mb16[p], (size_t)B * L * m * d * 2});
      pieces.push_back({(void**)&M->mss[p], (size_t)B * L * m * nc * 4});
    }
    pieces.push_back({(void**)&M->hss, rows * nc * 4});
    pieces.push_back({(void**)&M->rinv, rows * 4});
  }
  return pieces;
}

size_t workspace_need(rmt_model* M, int B) { return carve(workspace_pieces(M, B), nullptr); }

// Point the workspace pieces into the bound buffer for the current batch, or
// mark the workspace unusable when the buffer is too small for it.
void carve_workspace(rmt_model* M) {
  const std::vector<Piece> pieces = workspace_pieces(M, M->batch);
  M->ws_ok = M->ws != nullptr && carve(pieces, nullptr) <= M->ws_bytes;
  if (M->ws_ok) carve(pieces, M->ws);
}

// Pack the borrowed mathematical-layout weights into the bound weight buffer
// (on the model's stream; waits for the packing to finish).
int32_t pack_weights(rmt_model* M) {
  const rmt_config& c = M->cfg;
  const rmt_weights* w = &M->src;
  const int L = c.L, d = c.d, R = c.n + c.m;
  const size_t F = (size_t)c.ffn;
  const size_t NQ = has_attention(c) ? (size_t)nqkv(c) : 0;
  const size_t HQD = has_attention(c) ? (size_t)c.n_heads * c.head_dim : 0;
  hipStream_t st = M->stream;
  HIP_TRY(hipMemsetAsync(M->flag, 0, 256, st));
  if (c.cell == RMT_CELL_LINEAR_GELU) {
    HIP_TRY(hipMemcpyAsync(M->w32, w->w, (size_t)L * d * d * 4, hipMemcpyDeviceToDevice, st));
    HIP_TRY(hipMemcpyAsync(M->b32, w->b, (size_t)L * d * 4, hipMemcpyDeviceToDevice, st));
  } else if (c.cell == RMT_CELL_ENCODER) {
    const int bf = w->weight_dtype == RMT_BF16;
    HIP_TRY(launch_pack(L, d, (int)F, w->w1, nullptr, bf, PACK_PLAIN, M->wgu, st));
    HIP_TRY(launch_pack(L, (int)F, d, w->w2, nullptr, bf, PACK_PLAIN, M->wd, st));
    HIP_TRY(launch_pack(L, d, (int)NQ, w->wqkv, nullptr, bf, PACK_PLAIN, M->wqkv, st));
    HIP_TRY(launch_pack(L, (int)HQD, d, w->wo, nullptr, bf, PACK_PLAIN, M->wo, st));
    const size_t Ld4 = (size_t)L * d * 4;
    HIP_TRY(hipMemcpyAsync(M->g1, w->g1, Ld4, hipMemcpyDeviceToDevice, st));
    HIP_TRY(hipMemcpyAsync(M->beta1, w->beta1, Ld4, hipMemcpyDeviceToDevice, st));
    HIP_TRY(hipMemcpyAsync(M->g2, w->g2, Ld4, hipMemcpyDeviceToDevice, st));
    HIP_TRY(hipMemcpyAsync(M->beta2, w->beta2, Ld4, hipMemcpyDeviceToDevice, st));
    HIP_TRY(hipMemcpyAsync(M->bqkv, w->bqkv, (size_t)L * NQ * 4, hipMemcpyDeviceToDevice, st));
    HIP_TRY(hipMemcpyAsync(M->bo, w->bo, Ld4, hipMemcpyDeviceToDevice, st));
    HIP_TRY(hipMemcpyAsync(M->b1, w->b1, (size_t)L * F * 4, hipMemcpyDeviceToDevice, st));
    HIP_TRY(hipMemcpyAsync(M->b2, w->b2, Ld4, hipMemcpyDeviceToDevice, st));
  } else {
    const int bf = w->weight_dtype == RMT_BF16;
    const int f16 = c.dtype == RMT_F16;   // operands packed as fp16
    HIP_TRY(launch_pack(L, d, (int)F, w->wg, w->wu, bf, PACK_GATE_UP, M->wgu, st, f16));
    HIP_TRY(launch_pack(L, (int)F, d, w->wd, nullptr, bf, PACK_PLAIN, M->wd, st, f16));
    HIP_TRY(hipMemcpyAsync(M->g2, w->g2, (size_t)L * d * 4, hipMemcpyDeviceToDevice, st));
    if (c.cell == RMT_CELL_LLAMA) {
      // 128-wide heads: Q and K columns in rotation-pair groups of 64, so that
      // the QKV epilogue rotates within any 64-column wave tile
      const int rot = (c.n_heads + c.n_kv_heads) * c.head_dim;
      HIP_TRY(launch_pack(L, d, (int)NQ, w->wqkv, nullptr, bf, c.head_dim == 128 ? PACK_ROPE_PAIRS : PACK_PLAIN,
                          M->wqkv, st, f16, c.head_dim == 128 ? rot : 0));
      HIP_TRY(launch_pack(L, (int)HQD, d, w->wo, nullptr, bf, PACK_PLAIN, M->wo, st, f16));
      HIP_TRY(hipMemcpyAsync(M->g1, w->g1, (size_t)L * d * 4, hipMemcpyDeviceToDevice, st));
      // RoPE table: angle p * theta^(-2i/hd) in double precision.
      const int half = c.head_dim / 2;
      std::vector<float2> tab((size_t)R * half);
      for (int p = 0; p < R; ++p)
        for (int i = 0; i < half; ++i) {
          const double ang = (double)p * std::pow((double)c.rope_theta, -2.0 * i / c.head_dim);
          tab[(size_t)p * half + i] = make_float2((float)std::cos(ang), (float)std::sin(ang));
        }
      HIP_TRY(hipMemcpyAsync(M->rope, tab.data(), tab.size() * sizeof(float2), hipMemcpyHostToDevice, st));
      HIP_TRY(hipStreamSynchronize(st));   // `tab` is host memory of this frame
    }
  }
  HIP_TRY(hipStreamSynchronize(st));
  return RMT_OK;
}

int32_t check_forward_args(rmt_model* M, const void* tokens, const void* mem0, const rmt_output* out) {
  if (!M) return fail(RMT_EINVAL, "model is NULL");
  if (!tokens || !mem0 || !out || !out->hidden || !out->mem)
    return fail(RMT_EINVAL, "tokens, mem0, out, out->hidden and out->mem must be non-NULL");
  if (!M->wbuf) return fail(RMT_EWORKSPACE, "no weight buffer bound (rmt_model_bind, RMT_BUF_WEIGHTS)");
  if (!M->ws_ok)
    return fail(RMT_EWORKSPACE, "no workspace bound for a batch of %d (rmt_model_bind, RMT_BUF_WORKSPACE; "
                "%zu bytes needed, %zu bound)", M->batch, workspace_need(M, M->batch), M->ws_bytes);
  return RMT_OK;
}

int32_t start_forward(rmt_model* M, const void* mem0, const rmt_output* out) {
  const rmt_config& c = M->cfg;
  const size_t mem_bytes = (size_t)M->batch * c.L * c.m * c.d * sizeof(float);
  // M(l, -1) lives in the buffer that segment -1 maps to (see the header).
  float* dst = ((c.S - 1 - (-1)) % 2 == 0) ? out->mem : M->memw;
  M->cur_groups = 0;
  MARK(-1, 0.0, 0.0);
  if ((const void*)dst != mem0) {
    HIP_TRY(hipMemcpyAsync(dst, mem0, mem_bytes, hipMemcpyDeviceToDevice, M->stream));
    MARK(RMT_STAGE_GATHER, 0.0, 2.0 * mem_bytes);
  }
  if (c.cell == RMT_CELL_LLAMA) {
    // RMSNorm-1 inputs of M(l, -1): 16-bit copies y * g1[l] and chunk sums
    const int par = (c.S % 2 == 0) ? 0 : 1;     // the parity of segment -1
    const int rows = M->batch * c.L * c.m;
    HIP_TRY(launch_norm_aux_rows(rows, c.d, dst, c.m, c.L, 0, M->g1, M->mb16[par], M->mss[par],
                                 c.dtype == RMT_F16, M->stream));
    MARK(RMT_STAGE_GATHER, 0.0, (double)rows * c.d * 6 + (double)rows * (c.d / kChunk) * 4);
  }
  return RMT_OK;
}

// Queue every diagonal of the sweep: per diagonal, the regular cells in
// launches of up to kMaxGroups (layer-major, sequence fastest), then the cells
// of a short last segment in launches of their own.  Uses no heap memory.
int32_t sweep_diagonals(rmt_model* M, const void* tokens, const rmt_output* out) {
  const int L = M->cfg.L, S = M->cfg.S, B = M->batch;
  const bool ragged = M->n_last != M->cfg.n;
  Cell chunk[kMaxGroups];
  for (int k = 0; k < L + S - 1; ++k) {
    const int l_lo = std::max(0, k - S + 1), l_hi = std::min(L - 1, k);
    for (int pass = 0; pass < 2; ++pass) {      // 0: regular cells, 1: short cells
      int G = 0;
      for (int l = l_lo; l <= l_hi; ++l) {
        const bool short_cell = ragged && k - l == S - 1;
        if (short_cell != (pass == 1)) continue;
        for (int b = 0; b < B; ++b) {
          chunk[G++] = Cell{l, k - l, b};
          if (G == kMaxGroups) {
            const int32_t rc = run_cells(M, chunk, G, tokens, out);
            if (rc != RMT_OK) return rc;
            G = 0;
          }
        }
      }
      if (G > 0) {
        const int32_t rc = run_cells(M, chunk, G, tokens, out);
        if (rc != RMT_OK) return rc;
      }
    }
  }
  return RMT_OK;
}

// Device address of `scratch` on each device, looked up once per device (with
// that device current) and kept: in host code the array's name is only a
// host-side stand-in, never a device address.
std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;   // by device ordinal; nullptr until looked up

int32_t scratch_address(void** out) {
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (dev < 0) return fail(RMT_EHIP, "hipGetDevice returned %d", dev);
  if ((size_t)dev >= g_scratch_ptr.size()) g_scratch_ptr.resize((size_t)dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(RMT_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return RMT_OK;
}

}  // namespace

extern "C" {

const char* rmt_last_error(void) { return g_last_error.c_str(); }

int32_t rmt_diag_schedule(int32_t L, int32_t S, int32_t* diag_ptr, int32_t* cells) {
  if (L < 1 || S < 1) return fail(RMT_EINVAL, "L and S must be >= 1 (got %d, %d)", L, S);
  if ((int64_t)L * S > INT32_MAX || (int64_t)L + S > INT32_MAX)
    return fail(RMT_EINVAL, "L*S overflows int32");
  const int32_t ndiag = L + S - 1;
  if (!diag_ptr && !cells) return ndiag;
  if (!diag_ptr || !cells) return fail(RMT_EINVAL, "diag_ptr and cells must both be NULL or both set");
  int32_t idx = 0;
  diag_ptr[0] = 0;
  for (int32_t k = 0; k < ndiag; ++k) {
    const int32_t l_lo = std::max(0, k - S + 1), l_hi = std::min(L - 1, k);
    int32_t slot = 0;
    for (int32_t l = l_lo; l <= l_hi; ++l, ++slot, ++idx) {
      cells[3 * idx + 0] = l;
      cells[3 * idx + 1] = k - l;
      cells[3 * idx + 2] = slot;
    }
    diag_ptr[k + 1] = idx;
  }
  return ndiag;
}

int32_t rmt_model_create(const rmt_config* cfg, const rmt_weights* w, void* stream,
                         rmt_model** out) {
  if (!out) return fail(RMT_EINVAL, "out is NULL");
  *out = nullptr;
  int32_t rc = validate_config(cfg);
  if (rc != RMT_OK) return rc;
  if (!w) return fail(RMT_EINVAL, "weights are NULL");
  const rmt_config& c = *cfg;
  if (c.cell == RMT_CELL_LINEAR_GELU) {
    if (!w->w || !w->b) return fail(RMT_EINVAL, "LINEAR_GELU needs w and b");
    if (w->weight_dtype != RMT_F32) return fail(RMT_EUNSUPPORTED, "LINEAR_GELU weights must be fp32");
  } else if (c.cell == RMT_CELL_ENCODER) {
    if (!w->g1 || !w->beta1 || !w->wqkv || !w->bqkv || !w->wo || !w->bo || !w->g2 || !w->beta2 ||
        !w->w1 || !w->b1 || !w->w2 || !w->b2)
      return fail(RMT_EINVAL, "ENCODER needs g1, beta1, wqkv, bqkv, wo, bo, g2, beta2, w1, b1, w2, b2");
    if (w->weight_dtype != RMT_F32 && w->weight_dtype != RMT_BF16)
      return fail(RMT_EINVAL, "weight_dtype must be RMT_F32 or RMT_BF16");
  } else {
    if (!w->g2 || !w->wg || !w->wu || !w->wd) return fail(RMT_EINVAL, "g2, wg, wu and wd are required");
    if (c.cell == RMT_CELL_LLAMA && (!w->g1 || !w->wqkv || !w->wo || !w->embed))
      return fail(RMT_EINVAL, "LLAMA needs g1, wqkv, wo and embed");
    if (w->weight_dtype != RMT_F32 && w->weight_dtype != RMT_BF16)
      return fail(RMT_EINVAL, "weight_dtype must be RMT_F32 or RMT_BF16");
  }
  // No device work and no device memory: the weights stay where the caller
  // keeps them until rmt_model_bind packs them into the caller's buffer.
  rmt_model* M = new rmt_model();
  M->cfg = c;
  M->n_last = c.n;
  M->stream = (hipStream_t)stream;
  M->src = *w;
  M->embed = (const uint16_t*)w->embed;
  *out = M;
  return RMT_OK;
}

int32_t rmt_workspace_bytes(const rmt_model* model, int32_t kind, size_t* bytes) {
  if (!model || !bytes) return fail(RMT_EINVAL, "model and bytes must be non-NULL");
  rmt_model* M = const_cast<rmt_model*>(model);
  // size queries only: carve() writes no pointer when the base is NULL
  if (kind == RMT_BUF_WEIGHTS) *bytes = carve(weight_pieces(M), nullptr);
  else if (kind == RMT_BUF_WORKSPACE) *bytes = workspace_need(M, M->batch);
  else return fail(RMT_EINVAL, "kind must be RMT_BUF_WEIGHTS or RMT_BUF_WORKSPACE (got %d)", kind);
  return RMT_OK;
}

int32_t rmt_model_bind(rmt_model* M, int32_t kind, void* buffer, size_t bytes) {
  if (!M) return fail(RMT_EINVAL, "model is NULL");
  if (kind != RMT_BUF_WEIGHTS && kind != RMT_BUF_WORKSPACE)
    return fail(RMT_EINVAL, "kind must be RMT_BUF_WEIGHTS or RMT_BUF_WORKSPACE (got %d)", kind);
  if (!buffer) return fail(RMT_EINVAL, "buffer is NULL");
  if ((uintptr_t)buffer % 256 != 0) return fail(RMT_EINVAL, "buffer must be 256-byte aligned");
  if (kind == RMT_BUF_WEIGHTS) {
    if (M->wbuf) return fail(RMT_EINVAL, "the weights are already packed into a bound buffer");
    const std::vector<Piece> pieces = weight_pieces(M);
    const size_t need = carve(pieces, nullptr);
    if (bytes < need) return fail(RMT_EWORKSPACE, "weight buffer of %zu bytes, %zu needed", bytes, need);
    carve(pieces, buffer);
    M->wbuf = buffer;
    M->wbuf_bytes = bytes;
    const int32_t rc = pack_weights(M);
    if (rc != RMT_OK) {
      M->wbuf = nullptr;
      M->wbuf_bytes = 0;
      return rc;
    }
    // only the embedding is read after packing
    const void* embed = M->src.embed;
    M->src = rmt_weights{};
    M->src.embed = embed;
    return RMT_OK;
  }
  const size_t need = workspace_need(M, M->batch);
  if (bytes < need)
    return fail(RMT_EWORKSPACE, "workspace of %zu bytes, %zu needed for a batch of %d", bytes, need, M->batch);
  M->ws = buffer;
  M->ws_bytes = bytes;
  carve_workspace(M);
  return RMT_OK;
}

int32_t rmt_model_set_segments(rmt_model* model, int32_t S) {
  if (!model) return fail(RMT_EINVAL, "model is NULL");
  if (S < 1) return fail(RMT_EINVAL, "S must be >= 1");
  rmt_config c = model->cfg;
  c.S = S;
  int32_t rc = validate_config(&c);
  if (rc != RMT_OK) return rc;
  model->cfg.S = S;
  model->n_last = model->cfg.n;
  return RMT_OK;
}

int32_t rmt_model_set_tokens(rmt_model* model, int64_t T) {
  if (!model) return fail(RMT_EINVAL, "model is NULL");
  if (T < 1) return fail(RMT_EINVAL, "T must be >= 1");
  const int64_t n = model->cfg.n;
  const int64_t S = (T + n - 1) / n;
  if (S > INT32_MAX) return fail(RMT_EINVAL, "T is too large");
  rmt_config c = model->cfg;
  c.S = (int32_t)S;
  int32_t rc = validate_config(&c);
  if (rc != RMT_OK) return rc;
  model->cfg.S = (int32_t)S;
  model->n_last = (int)(T - (S - 1) * n);
  return RMT_OK;
}

int32_t rmt_model_set_batch(rmt_model* model, int32_t B) {
  if (!model) return fail(RMT_EINVAL, "model is NULL");
  if (B < 1) return fail(RMT_EINVAL, "B must be >= 1 (got %d)", B);
  const rmt_config& c = model->cfg;
  if ((int64_t)B * c.S * c.n > ((int64_t)1 << 40) / std::max(1, c.d))
    return fail(RMT_EINVAL, "B * S * n * d is too large");
  model->batch = B;
  carve_workspace(model);   // keeps the bound workspace if it is large enough for B
  return RMT_OK;
}

int32_t rmt_model_set_stream(rmt_model* model, void* stream) {
  if (!model) return fail(RMT_EINVAL, "model is NULL");
  model->stream = (hipStream_t)stream;
  return RMT_OK;
}

int32_t rmt_model_device_bytes(const rmt_model* model, size_t* bytes) {
  if (!model || !bytes) return fail(RMT_EINVAL, "model and bytes must be non-NULL");
  *bytes = model->wbuf_bytes + model->ws_bytes;
  return RMT_OK;
}

int32_t rmt_forward_diagonal(rmt_model* M, const void* tokens, const void* mem0, rmt_output* out) {
  int32_t rc = check_forward_args(M, tokens, mem0, out);
  if (rc != RMT_OK) return rc;
  rc = start_forward(M, mem0, out);
  if (rc != RMT_OK) return rc;
  return sweep_diagonals(M, tokens, out);
}

int32_t rmt_forward_diagonal_static(rmt_model* M, const void* tokens, const void* mem0,
                                    rmt_output* out) {
  if (!M) return fail(RMT_EINVAL, "model is NULL");
  const size_t need = workspace_need(M, M->batch);
  if (need > kStaticScratchBytes)
    return fail(RMT_EWORKSPACE,
                "this model needs %zu bytes of workspace for a batch of %d; the static scratch of "
                "rmt_forward_diagonal_static holds %zu",
                need, M->batch, kStaticScratchBytes);
  void* base = nullptr;
  int32_t rc = scratch_address(&base);
  if (rc != RMT_OK) return rc;
  // The scratch stands in for the bound workspace during this call only.
  void* const ws = M->ws;
  const size_t ws_bytes = M->ws_bytes;
  const bool timing = M->timing;
  M->ws = base;
  M->ws_bytes = kStaticScratchBytes;
  M->timing = false;        // no event is created or recorded
  carve_workspace(M);
  rc = check_forward_args(M, tokens, mem0, out);
  if (rc == RMT_OK) rc = start_forward(M, mem0, out);
  if (rc == RMT_OK) rc = sweep_diagonals(M, tokens, out);
  M->ws = ws;
  M->ws_bytes = ws_bytes;
  M->timing = timing;
  carve_workspace(M);
  return rc;
}

int32_t rmt_forward_sequential(rmt_model* M, const void* tokens, const void* mem0, rmt_output* out) {
  int32_t rc = check_forward_args(M, tokens, mem0, out);
  if (rc != RMT_OK) return rc;
  rc = start_forward(M, mem0, out);
  if (rc != RMT_OK) return rc;
  for (int b = 0; b < M->batch; ++b)
    for (int s = 0; s < M->cfg.S; ++s)
      for (int l = 0; l < M->cfg.L; ++l) {
        Cell cell{l, s, b};
        rc = run_cells(M, &cell, 1, tokens, out);
        if (rc != RMT_OK) return rc;
      }
  return RMT_OK;
}

int32_t rmt_model_check(rmt_model* M, int32_t* bad_tokens) {
  if (!M || !bad_tokens) return fail(RMT_EINVAL, "model and bad_tokens must be non-NULL");
  if (!M->wbuf) return fail(RMT_EWORKSPACE, "no weight buffer bound");
  int32_t v = 0;
  HIP_TRY(hipMemcpyAsync(&v, M->flag, sizeof(v), hipMemcpyDeviceToHost, M->stream));
  HIP_TRY(hipStreamSynchronize(M->stream));
  HIP_TRY(hipMemsetAsync(M->flag, 0, sizeof(v), M->stream));
  HIP_TRY(hipStreamSynchronize(M->stream));
  *bad_tokens = v ? 1 : 0;
  return RMT_OK;
}

int32_t rmt_model_enable_timing(rmt_model* M, int32_t enable) {
  if (!M) return fail(RMT_EINVAL, "model is NULL");
  M->timing = enable != 0;
  M->ev_used = 0;
  M->ev_stage.clear();
  M->ev_flops.clear();
  M->ev_bytes.clear();
  M->ev_groups.clear();
  return RMT_OK;
}

namespace {

// Per-stage sums over the recorded launches that covered g_lo..g_hi cells.
int32_t sum_stage_times(rmt_model* M, int g_lo, int g_hi, double* ms, int64_t* launches,
                        double* flops, double* bytes) {
  HIP_TRY(hipStreamSynchronize(M->stream));
  double t[RMT_NUM_STAGES] = {0}, f[RMT_NUM_STAGES] = {0}, b[RMT_NUM_STAGES] = {0};
  int64_t nl[RMT_NUM_STAGES] = {0};
  for (size_t i = 1; i < M->ev_used; ++i) {
    const int st = M->ev_stage[i];
    if (st < 0) continue;   // start marker of the next forward call
    if (M->ev_groups[i] < g_lo || M->ev_groups[i] > g_hi) continue;
    float dt = 0.f;
    HIP_TRY(hipEventElapsedTime(&dt, M->events[i - 1], M->events[i]));
    t[st] += dt;
    nl[st] += 1;
    f[st] += M->ev_flops[i];
    b[st] += M->ev_bytes[i];
  }
  for (int i = 0; i < RMT_NUM_STAGES; ++i) {
    if (ms) ms[i] = t[i];
    if (launches) launches[i] = nl[i];
    if (flops) flops[i] = f[i];
    if (bytes) bytes[i] = b[i];
  }
  return RMT_OK;
}

}  // namespace

int32_t rmt_model_stage_times(rmt_model* M, double* ms, int64_t* launches, double* flops,
                              double* bytes) {
  if (!M) return fail(RMT_EINVAL, "model is NULL");
  const int32_t rc = sum_stage_times(M, INT32_MIN, INT32_MAX, ms, launches, flops, bytes);
  if (rc != RMT_OK) return rc;
  M->ev_used = 0;
  M->ev_stage.clear();
  M->ev_flops.clear();
  M->ev_bytes.clear();
  M->ev_groups.clear();
  return RMT_OK;
}

int32_t rmt_model_stage_times_groups(rmt_model* M, int32_t g_lo, int32_t g_hi, double* ms,
                                     int64_t* launches, double* flops, double* bytes) {
  if (!M) return fail(RMT_EINVAL, "model is NULL");
  if (g_lo > g_hi) return fail(RMT_EINVAL, "g_lo (%d) > g_hi (%d)", g_lo, g_hi);
  return sum_stage_times(M, g_lo, g_hi, ms, launches, flops, bytes);
}

int32_t rmt_model_destroy(rmt_model* M) {
  if (!M) return RMT_OK;
  // The bound buffers belong to the caller: nothing to free on the device.
  // Device work is queued only once the weights are bound (packing, forward
  // calls), so a model without them has nothing to wait for.
  hipError_t e1 = M->wbuf ? hipStreamSynchronize(M->stream) : hipSuccess;
  for (hipEvent_t e : M->events) (void)hipEventDestroy(e);
  delete M;
  if (e1 != hipSuccess) return fail(RMT_EHIP, "hipStreamSynchronize: %s", hipGetErrorString(e1));
  return RMT_OK;
}

int32_t rmt_pack_weight(int32_t L, int32_t K, int32_t N, const void* src, int32_t src_dtype,
                        void* dst, void* stream) {
  if (L < 1 || K < 1 || N < 1 || K % 8 != 0 || N % 8 != 0)
    return fail(RMT_EINVAL, "need L >= 1 and positive K, N that are multiples of 8");
  if (!src || !dst) return fail(RMT_EINVAL, "src and dst must be non-NULL");
  if (src_dtype != RMT_F32 && src_dtype != RMT_BF16) return fail(RMT_EINVAL, "bad src_dtype");
  HIP_TRY(launch_pack(L, K, N, src, nullptr, src_dtype == RMT_BF16, PACK_PLAIN, (uint16_t*)dst,
                      (hipStream_t)stream));
  return RMT_OK;
}

int32_t rmt_grouped_gemm(int32_t G, int32_t Mr, int32_t N, int32_t K, int32_t Lw, const void* A,
                         const void* B, const int32_t* group_layer, void* C, int32_t dtype, void* stream) {
  if (G < 1 || G > kMaxGroups) return fail(RMT_EINVAL, "G must be in [1, %d] (got %d)", kMaxGroups, G);
  if (Mr < 1 || K < 8 || K % 8 != 0 || N < 64 || N % 64 != 0)
    return fail(RMT_EINVAL, "need M >= 1, K a positive multiple of 8, N a positive multiple of 64");
  if (Lw < 1) return fail(RMT_EINVAL, "Lw must be >= 1 (got %d)", Lw);
  if ((int64_t)G * Mr * std::max(N, K) > INT32_MAX) return fail(RMT_EINVAL, "sizes overflow int32");
  if (!A || !B || !C || !group_layer) return fail(RMT_EINVAL, "A, B, C and group_layer must be non-NULL");
  if (dtype != RMT_BF16 && dtype != RMT_F16)
    return fail(RMT_EUNSUPPORTED, "dtype must be RMT_BF16 or RMT_F16 (got %d)", dtype);
  for (int g = 0; g < G; ++g)
    if (group_layer[g] < 0 || group_layer[g] >= Lw)
      return fail(RMT_EINVAL, "group_layer[%d] = %d is outside [0, %d)", g, group_layer[g], Lw);
  GroupTable tab;
  std::memset(&tab, 0, sizeof(tab));
  tab.G = G;
  for (int g = 0; g < G; ++g) {
    tab.layer[g] = group_layer[g];
    tab.out_lo[g] = (uint16_t*)C + (size_t)g * Mr * N;
  }
  GemmArgs ga;
  std::memset(&ga, 0, sizeof(ga));
  ga.A = (const uint16_t*)A; ga.B = (const uint16_t*)B; ga.M = Mr; ga.N = N; ga.K = K;
  ga.split_in = Mr; ga.split_out = Mr; ga.ld_out = N; ga.f16 = dtype == RMT_F16;
  HIP_TRY(launch_gemm(EPI_STORE_BF16, ga, tab, (hipStream_t)stream));
  return RMT_OK;
}

int32_t rmt_attention(int32_t G, int32_t R, int32_t Hq, int32_t Hkv, int32_t hd, int32_t causal,
                      const void* qkv, void* out, void* stream) {
  if (G < 1 || G > 65535 || R < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
    return fail(RMT_EINVAL, "need 1 <= G <= 65535, R >= 1 and n_heads a multiple of n_kv_heads");
  if (!qkv || !out) return fail(RMT_EINVAL, "qkv and out must be non-NULL");
  if (hd != 64 && hd != 128) return fail(RMT_EUNSUPPORTED, "head_dim must be 64 or 128");
  if (!head_ratio_ok(Hq, Hkv))
    return fail(RMT_EUNSUPPORTED, "n_heads / n_kv_heads must be 1, 2 or a multiple of 4");
  if ((int64_t)G * R * (Hq + 2 * Hkv) * hd > ((int64_t)1 << 40)) return fail(RMT_EINVAL, "sizes too large");
  if ((int64_t)R * (Hq + 2 * Hkv) * hd * 2 > INT32_MAX)
    return fail(RMT_EINVAL, "one cell's qkv rows must stay below 2 GiB (32-bit buffer offsets)");
  HIP_TRY(launch_attention((const uint16_t*)qkv, (uint16_t*)out, G, R, Hq, Hkv, hd, causal != 0, false,
                           (hipStream_t)stream));
  return RMT_OK;
}

int32_t rmt_causal_attention(int32_t G, int32_t R, int32_t Hq, int32_t Hkv, int32_t hd,
                             const void* qkv, void* out, void* stream) {
  return rmt_attention(G, R, Hq, Hkv, hd, 1, qkv, out, stream);
}

}  // extern "C"
