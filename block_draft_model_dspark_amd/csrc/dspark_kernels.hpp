// Kernel argument blocks and launchers of the gfx950 DSpark draft round.
// Arguments travel by value (kernarg segment), so per-row tables are bounded:
// at most MAX_ROWS draft rows per round.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsp {

enum { WK_F32 = 0, WK_BF16 = 1, WK_Q4 = 2 };   // weight storage kinds
enum { XM_F32 = 0, XM_BF16 = 1, XM_NORM = 2 };  // how a GEMM reads its input rows

constexpr int MAX_ROWS = 64;
constexpr int MAX_SEG = 8;
constexpr int MAX_LAYERS = 64;
constexpr int WALK_CHUNK = 64;  // vocabulary entries per walk-statistics chunk (one GEMM column block)
constexpr int ATT_KEYS = 32;    // keys staged per attention pass

// Row statistics of one 64-column block of a sublayer output y with the
// residual h it is added to and the norm weight w1 of that sum:
// (sum y^2, sum h*w1*y, sum (w1*y)^2, sum h^2).  Enough to form both RMSNorm
// factors of the sandwich  hn = (h + rms(y)*w1) * sc,  x = rms(hn) * w2
// without another pass over the row.  The sum of hn^2 is formed as
// sc^2 (S_hh + 2 r1 S_hwy + r1^2 S_wywy), which cancels when the normed
// sublayer output nearly cancels the residual: the products and sums are
// therefore taken in fp64 (a product of two fp32 values is exact there), so
// the combination keeps its accuracy down to cancellations of ~1e8.
struct RowStats {
  double x, y, z, w;  // sum y^2, sum h w1 y, sum (w1 y)^2, sum h^2
};

// the sandwich's two RMS factors from a row's summed statistics over K
// columns: r1 = rms factor of y, r2 = rms factor of hn = (h + r1 w1 y) sc
__host__ __device__ inline float2 norm_factors(const RowStats& s, float sc, int K, float eps) {
  const double r1 = 1.0 / sqrt(s.x / K + (double)eps);
  const double t2 = (double)sc * sc * (s.w + 2.0 * r1 * s.y + r1 * r1 * s.z);
  const double r2 = 1.0 / sqrt((t2 > 0.0 ? t2 : 0.0) / K + (double)eps);
  return make_float2((float)r1, (float)r2);
}

struct NormIn {
  const float* h;      // [M, K] residual, or null (zero)
  const float* y;      // [M, K] sublayer output, or null (zero)
  const RowStats* sums;  // [nparts, M] statistics of 64-column blocks
  int nparts;          // K / 64
  const void* w1;      // [K] act dtype (unused when y is null)
  const void* w2;      // [K] act dtype, or null: x = hn
  const float* sc;     // [1] fp32 residual scale (a layer_scalar copy), or null: 1
  float* hout;         // [M, K]: hn is written here by column block 0, or null
  int64_t ld;          // row pitch (floats) of h, y and hout
  float eps;
  int act_bf16;
};

// y[m, n] partials of a GEMM x[M, K] . W[N, K]^T over K slices:
// P[s][m][n], s = blockIdx.y.  Output columns [seg[i].n0, seg[i+1].n0) read
// weight segment i at row n - seg[i].n0 (segments are 16-column aligned).
struct GemmSeg {
  const void* w;      // f32 / bf16 [rows, K], or q4 packed uint32 [rows, K/8]
  const void* s;      // q4 scales bf16 [rows, K/64]
  const void* b;      // q4 biases bf16 [rows, K/64]
  int n0;
  int pad_;
};
struct GemmArgs {
  const void* X;      // XM_F32: [M, ldx] f32; XM_BF16: [M, ldx] bf16; XM_NORM: see nin
  int64_t ldx;
  int M, N, K;        // N a multiple of 64
  int kslice;         // K range per blockIdx.y
  int kc;             // K sub-slice staged per iteration
  int nseg;
  GemmSeg seg[MAX_SEG];
  float* P;           // split-K partials (S > 1): S x ceil(M/16) x (N/64) tiles of 16 x 64 fp32
  NormIn nin;
};

// what the GEMM does with its result (see dspark_gemm.hip)
enum { EPI_Y = 0, EPI_QK = 1, EPI_GELU = 2, EPI_SUMS = 3, EPI_LM = 4, EPI_KV = 5 };

// ---- address arithmetic shared by the kernels and the host ----------------
// (host code replays the 4-bit kernels' addresses with these: see
// dspark_q4_address_check)
//
// 4-bit storage, eight codes per uint32 word and groups of `group` codes
// along each row: the word holding element (row, k) of a [rows, cols]
// matrix, and the index of its scale / bias
__host__ __device__ inline int64_t q4_word(int64_t row, int cols, int k) { return row * (cols >> 3) + (k >> 3); }
__host__ __device__ inline int64_t q4_group(int64_t row, int cols, int group, int k) {
  return row * (cols / group) + k / group;
}
// streaming GEMM: the first of the two words lane group gq loads for the j-th
// 64-wide group of the sub-slice that starts at kc (codes kc + 64j + 16gq ..
// kc + 64j + 16gq + 15 of weight row wrow), and that group's scale / bias
__host__ __device__ inline int64_t q4_gemm_word(int64_t wrow, int K, int kc, int gq, int j) {
  return q4_word(wrow, K, kc) + 2 * gq + 8 * j;
}
__host__ __device__ inline int64_t q4_gemm_group(int64_t wrow, int K, int kc, int j) {
  return q4_group(wrow, K, 64, kc) + j;
}
// streaming GEMM staging buffer of one sub-slice of kc: the bf16 activation
// planes (one for bf16 rows, hi and lo otherwise) of mt 16-row tiles, then,
// for 4-bit weights, the per-(row, 64-group) activation sums
__host__ __device__ constexpr size_t xsum_offset(int xmode, int mt, int kc) {
  return (size_t)mt * (kc / 32) * 64 * 16 * (xmode == XM_BF16 ? 1 : 2);
}
__host__ __device__ constexpr size_t xbuf_bytes(int wkind, int xmode, int mt, int kc) {
  return xsum_offset(xmode, mt, kc) + (wkind == WK_Q4 ? (size_t)mt * 16 * (kc / 64) * 4 : 0);
}
// first output column of wave w in column block c.  gate|up: waves 0,1 take
// gate columns 32c.., waves 2,3 the matching up columns.  q|k heads: waves
// 0,1 take head dims [32c', 32c'+32), waves 2,3 their RoPE partners + hd/2
// (c' = c mod hd/64), so a workgroup holds whole rotation pairs.
template <int EPI>
__host__ __device__ inline int wave_col(int c, int w, int N, int hd) {
  if constexpr (EPI == EPI_GELU) return (w >> 1) * (N >> 1) + 32 * c + 16 * (w & 1);
  if constexpr (EPI == EPI_QK) {
    const int hj = hd >> 6, head = c / hj, cp = c - head * hj;
    return head * hd + (w >> 1) * (hd >> 1) + 32 * cp + 16 * (w & 1);
  }
  return 64 * c + 16 * w;
}

struct RopeCfg {
  double step;        // theta^(-2 / hd): 1 / wavelength of pair k is step^k
  int hd, nrot;       // rotated pairs: k < nrot turn, the rest pass through
};

// Sampling at temperature > 0 (see dspark.h, dspark_draft_args): the
// logits epilogue also writes zs = z + T g, g the Gumbel noise of row
// m / gamma's key stream at slot m mod gamma, and forms the walk's chunk
// bounds on zs, so the greedy walk over zs draws from softmax(u / T)
struct SampleArgs {
  float temperature;  // <= 0: no sampling
  int gamma;
  float* zs;          // [M, V]; may equal the logits buffer (then only zs is stored)
  uint64_t seeds[MAX_ROWS];
};

struct EpiArgs {
  float* Y;           // [M, N] fp32 result (EPI_Y, EPI_SUMS, EPI_LM, EPI_KV)
  unsigned* cnt;      // reduction counters, zero on entry, left zero
  int group_cols;     // EPI_KV: columns per head group
  float eps;
  int act_bf16;
  // EPI_QK / EPI_KV
  int nH, nKv, hd, gamma;
  const float2* rt;   // EPI_QK: [rows, hd/2] (cos, sin) of each row's position and pair
  const void* qn; const void* kn;
  float* q;           // [A, nKv, nq, hd] RoPE(q_norm_w * y), nq = (nH/nKv)*gamma, row hl*gamma + g
  float* kb;          // [A, nKv, gamma, hd] RoPE(k_norm_w * y)
  float* vb;          // [A, nKv, gamma, hd] y
  float* ssq;         // [(nH+nKv) * hd/64, M] sum y^2 per head and 64-column part
  int L;              // EPI_KV: context rows per batch row
  RopeCfg rope;       // EPI_KV: RoPE of position pos0[b] + i for row b * L + i
  int pos0[MAX_ROWS];
  const void* kn_l[MAX_SEG];
  void* kout[MAX_SEG]; void* vout[MAX_SEG];  // [B, nKv, L, hd] act dtype
  // EPI_KV on the weight-streaming kernel without split K: store the product
  // to Y and leave the norms and RoPE to a separate k_kv_epi launch (no
  // cross-workgroup arrival, so no counters)
  int kv_defer;
  // EPI_GELU
  float* act;         // [M, N/2], row pitch ld_act
  int64_t ld_act;
  uint16_t* act_planes;  // tiled gate|up only: act as bf16 hi / lo planes (see TallArgs)
  int64_t act_plane;
  // EPI_SUMS
  int64_t ldy;        // row pitch (floats) of Y and h
  const float* h;     // residual [M, N] or null
  const void* w1;     // norm weight [N]
  RowStats* sums;     // [N/64, M]
  // EPI_LM
  float cap;          // <= 0: none
  const float* aux;   // [V] markov_w2 row norms, aux[V] = max markov_w1 row norm; null when rank 0
  float2* lohi;       // [M, NC] (max z - B, max z + B) per chunk
  int NC;
  SampleArgs smp;
};

// tiled GEMM over many rows (dspark_tall.hip): T[m, n] = sum over the np
// bf16 input planes X_p[m, :] . W[n, :], fp32, row pitch ldt
enum { TALL_NONE = 0, TALL_64 = 1, TALL_128 = 2 };  // output tile (square)
struct TallArgs {
  const uint16_t* X;  // plane 0 [M, ldx] bf16; plane p at X + p * plane
  int64_t ldx, plane;
  int M, N, K;        // K a multiple of 64
  int nseg;
  GemmSeg seg[MAX_SEG];  // bf16 weights [rows, K] per column segment
  int kslice;         // K range per blockIdx.z (a multiple of 64)
  float* T;           // partial product of slice z at T + z * tstride
  int64_t ldt, tstride;
  // logits in the tiled kernel itself (128 x 128 tiles, one K slice): T
  // holds z = cap tanh(x / cap) (cap 0: x), and lohi[m, c] = (max z - B,
  // max z + B) over the 64 vocabulary entries of chunk c, B the walk bound
  // of each entry (aux null: 0)
  int lm;
  float cap;
  const float* aux;
  float2* lohi;       // [M, NC]
  int NC;
  // gate|up in the tiled kernel itself (128 x 128 tiles, hi + lo planes, one
  // K slice): tile x multiplies gate rows 64x.. and up rows I + 64x.. (N = 2I)
  // and writes act[m, 64x + c] = gelu_tanh(gate) * up
  int gelu;
  float* act;
  int64_t ld_act;
  // non-null: act goes out as the bf16 hi / lo planes [2][M, N/2] (plane
  // stride act_plane) that a tiled down projection reads, instead of fp32
  uint16_t* act_planes;
  int64_t act_plane;
};

// Tile order of the tiled GEMM: workgroups go round-robin over the 8 XCDs
// in launch order (linear id w runs on XCD w mod 8), and each XCD has its own
// L2.  Maps the linear workgroup id w of a gx x gy grid (column tiles x row
// tiles) to the output tile (bx, by) it computes:
//  - the weights are the big operand (at most 8 row tiles) and the column
//    tiles are a multiple of 8: XCD x takes the row tiles of column tile
//    x, x + 8, ... back to back, so they stream that weight tile through its
//    L2 together;
//  - more than 8 row tiles, a multiple of 8 (the activation rows are the big
//    operand): XCD x takes row tiles x, x + 8, ... each across every column
//    tile, so each activation row is read by one XCD only; when the column
//    tiles are a multiple of 8 too, against 8 column tiles at a time, so the
//    tiles in flight on the XCD share weight tiles as well;
//  - otherwise the plain order bx = w mod gx, by = w / gx.
// A bijection of [0, gx gy) onto the tiles in every case.
__host__ __device__ inline void tall_tile_of(int gx, int gy, int w, int& bx, int& by) {
  bx = w % gx;
  by = w / gx;
  const int s = w >> 3;
  if ((gx & 7) == 0 && gy <= 8) {
    bx = (s / gy) * 8 + (w & 7);
    by = s % gy;
  } else if ((gy & 7) == 0 && gy > 8) {
    if ((gx & 7) == 0) {
      const int R = gy >> 3, inner = s % (8 * R), outer = s / (8 * R);
      by = 8 * (inner >> 3) + (w & 7);
      bx = 8 * outer + (inner & 7);
    } else {
      by = (s / gx) * 8 + (w & 7);
      bx = s % gx;
    }
  }
}

// Block order of the weight-streaming GEMM (grid: gx column blocks x S K
// slices x R row blocks; workgroups are dealt to the 8 XCDs in launch order).
// In launch order the R row blocks of one (column block, K slice) are
// gx * S workgroups apart, so with several row blocks each weight tile would
// stream from HBM once per row block.  With R > 1 and gx * S a multiple of 8,
// workgroup (x, y, z) is renumbered so that XCD (x + gx y) mod 8 runs the R
// row blocks of its (column block, slice) pairs back to back and they share
// each weight tile in its L2.  A bijection of the (x, y, z) triples in every
// case.
__host__ __device__ inline void stream_block_of(int gx, int S, int R, int x, int y, int z, int& bx, int& by,
                                                int& bz) {
  bx = x;
  by = y;
  bz = z;
  const int units = gx * S;  // (column block, K slice) pairs
  if (R > 1 && (units & 7) == 0) {
    const int w = x + gx * y + units * z, s = w >> 3;
    const int u = (s / R) * 8 + (w & 7);
    bz = s % R;
    bx = u % gx;
    by = u / gx;
  }
}

// per-row data of a draft round
struct RowTab {
  int A, gamma;
  int anchor[MAX_ROWS];
  int pos[MAX_ROWS];  // block start position of each row
  int len[MAX_ROWS];  // context rows of each row
};

struct EmbedArgs {
  const void* E; const void* Es; const void* Eb; int ekind; int group;
  int H; float scale; int mask_id;
  int act_bf16, nL;
  const void* scal_src[MAX_LAYERS];  // per layer layer_scalar [1] act dtype
  float* scal;        // [nL + 1]: 1, then the layer scalars as fp32
  float* h;           // [M, H] scaled embedding rows, row pitch ldh
  int64_t ldh;
  RowStats* sums;     // [H/64, M] (0, 0, 0, sum h^2)
  float2* rt;         // [M, hd/2] RoPE table of the block positions
  RopeCfg rope;
  unsigned* cnt; int ncnt;  // GEMM counters zeroed here
  RowTab rows;
};

struct AttnRow {
  const void* k;      // [nKv, len, hd] act dtype
  const void* v;
};
struct AttnArgs {
  AttnRow row[MAX_ROWS];
  int len[MAX_ROWS];
  int split_off[MAX_ROWS + 1];  // prefix sum of key splits per row (context splits, then one block split)
  int A, gamma, nKv, nH, nq, split, M, hd;
  // wide kernel: 0 = workgroup x runs split x; else workgroup x runs slot
  // x / 8 of the splits of rows x mod 8, x mod 8 + 8, ... (workgroups are
  // dealt to the eight XCDs in turn, so all splits of a row share one L2 and
  // its query rows are fetched once), grid 8 * wide_slots
  int xcd_rows;
  float eps;
  const float* q; const float* kb; const float* vb; const float* ssq;
  // V-only context cache (row[a].k unused): the context keys are rebuilt as
  // K = RoPE(V * k_norm) at positions ctx_pos0[a] + j while they are staged
  int vonly;
  const void* kn;        // this layer's k_norm weight [hd], bf16
  double rope_step;      // theta^(-2 / hd)
  int nrot;
  int ctx_pos0[MAX_ROWS];
  // [nsplit, nKv, nq, hd]: fp32 unnormalised for an fp32 cache; for a bf16
  // cache, fp16 of O / sum (|O / sum| <= max |v|, unit-RMS value rows)
  void* opart;
  float* ml;          // [nsplit, nKv, nq, 2] (max, sum)
};

struct MergeArgs {
  int split_off[MAX_ROWS + 1];
  int A, gamma, nKv, nq, nH, hd;
  int part_f16;       // partials are fp16 O / sum (else fp32 unnormalised)
  int lane_order;     // fp16 partials in the wide attention's lane order (else [split, kvh, nq, hd])
  const void* opart; const float* ml;
  float* O;           // [A*gamma, nH*hd], row pitch ldo
  int64_t ldo;
  // non-null: O goes out as the bf16 hi / lo planes [2][A*gamma, nH*hd]
  // (plane stride `plane`) that the tiled o projection reads, instead of fp32
  uint16_t* planes;
  int64_t plane;
};

struct WalkArgs {
  RowTab rows;
  int V, NC, rank, wkind, group;
  const float* z; const float2* lohi; const float* aux;
  const void* w1; const void* w1s; const void* w1b;
  const void* w2; const void* w2s; const void* w2b;
  // RNN head: s_k = tanh(s_{k-1} wh + w1[prev] + bh), bias = w2 s_k
  int rnn, act_bf16;
  const void* wh; const void* whs; const void* whb;  // [rank, rank], weight dtype
  const void* bh;                                      // [rank], act dtype
  int32_t* tokens;
};

// deepspec.ts, #confidence and draftRows truncation (see k_conf)
constexpr int CONF_MAX_GAMMA = 32;
struct ConfArgs {
  RowTab rows;
  int H, rank, with_markov, wkind, group, act_bf16;
  int head;               // 0: no confidence head (lengths = gamma, conf untouched)
  const float* hn;        // [A*gamma, H] final residual rows (before the final norm), row pitch ldh
  int64_t ldh;
  const void* wnorm;      // final norm weight [H], act dtype
  float eps;
  const void* pw; const void* ps; const void* pb;  // proj weight [1, H (+ rank)] (q4: scales, biases)
  const void* bias;       // [1] act dtype
  const void* w1; const void* w1s; const void* w1b;  // markov_w1 [V, rank]
  const int32_t* tokens;  // [A, gamma] the walk's tokens
  float thr[CONF_MAX_GAMMA];  // per-slot thresholds; <= 0: slot not tested
  float* conf;            // [A, gamma]
  int32_t* lengths;       // [A] confident prefix lengths, or null
};

struct AuxArgs {
  int V, rank, wkind, group;
  const void* w1; const void* w1s; const void* w1b;
  const void* w2; const void* w2s; const void* w2b;
  float* aux;
  int rnn;  // aux[V] bounds the RNN state's norm (sqrt(rank)) instead of the markov_w1 rows'
};

// launchers (return hipGetLastError())
hipError_t launch_gemm(const GemmArgs& a, const EpiArgs& e, int epi, int wkind, int xmode, int mt, int S,
                       hipStream_t st);
size_t gemm_lds_bytes(int wkind, int xmode, int mt, int kc);
size_t gemm_counter_words(int M, int N, int mt, int group_cols);
hipError_t launch_xprep(const GemmArgs& g, int xmode, uint16_t* xop, int64_t plane, hipStream_t st);
// The split-K epilogue of a tiled o or down projection fused with the next
// GEMM's input preparation, one workgroup per row: y = sum of the S partial
// products, hn = (h + rms(y) w1 y) sc (written to hout when given), and the
// next GEMM's input x = rms(hn) w2 (x = hn without w2) as bf16 hi / lo planes.
// The whole row is in the workgroup, so both RMS factors come from direct
// fp64 sums of y^2 and hn^2.
constexpr int SP_KMAX = 8192;  // row width (a multiple of 8)
struct SumsPrepArgs {
  const float* T;     // partial products [S][M][ldt] (slice stride tstride)
  int64_t ldt, tstride;
  int S, M, K;
  const float* h;     // [M, ldh] residual, or null (zero)
  int64_t ldh;
  const void* w1;     // [K] act dtype: norm weight of y
  const float* sc;    // [1] residual scale, or null: 1
  const void* w2;     // [K] act dtype: the next input norm weight, or null
  int act_bf16;
  float eps;
  float* hout;        // [M, ldh] hn rows, or null
  uint16_t* xop;      // [2][M, K] bf16 hi / lo planes (plane stride `plane`)
  int64_t plane;
};
hipError_t launch_sums_prep(const SumsPrepArgs& a, hipStream_t st);
hipError_t launch_tall(const TallArgs& t, int tile, int np, int S, hipStream_t st);
// the epilogue of a GEMM whose product is the sum of S partial planes in T
// (row pitch ldt, plane stride tstride); EPI_KV reads it from e.Y (pitch N,
// S == 1)
hipError_t launch_gemm_epi(const GemmArgs& a, const EpiArgs& e, int epi, const float* T, int64_t ldt, int S,
                           int64_t tstride, hipStream_t st);
hipError_t launch_embed(const EmbedArgs& a, int M, hipStream_t st);
hipError_t launch_attn(const AttnArgs& a, bool kv_bf16, int nsplit, hipStream_t st);
// one workgroup per (row, split, kv head) with every query row (nq = 32, 64
// or 128 rows, staging layout permitting)
bool attn_wide_ok(int nq, int hd);
// whether the kernel that takes these shapes can rebuild context keys from a
// V-only cache (each staging thread must hold both halves of its RoPE pairs)
bool attn_vonly_ok(int nq, int hd, bool wide);
hipError_t launch_attn_wide(const AttnArgs& a, bool kv_bf16, int nsplit, hipStream_t st);
hipError_t launch_zero(unsigned* p, int64_t n, hipStream_t st);
hipError_t launch_merge(const MergeArgs& a, hipStream_t st);
hipError_t launch_walk(const WalkArgs& a, hipStream_t st);
hipError_t launch_aux(const AuxArgs& a, hipStream_t st);
hipError_t launch_conf(const ConfArgs& a, hipStream_t st);

}  // namespace dsp
