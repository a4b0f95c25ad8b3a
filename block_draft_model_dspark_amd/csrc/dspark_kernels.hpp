// Kernel argument blocks and launchers of the gfx950 DSpark draft round.
// Arguments travel by value (kernarg segment), so per-row tables are bounded:
// at most MAX_ROWS draft rows per round.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsp {

enum { WK_F32 = 0, WK_BF16 = 1, WK_Q4 = 2 };  // weight storage kinds

constexpr int MAX_ROWS = 64;
constexpr int MAX_SEG = 8;
constexpr int WALK_CHUNK = 256;  // vocabulary entries per walk-statistics chunk
constexpr int WALK_TOP = 4;      // best candidates kept per chunk

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
  const void* X;      // [M, ldx] f32, or bf16 when the X-is-bf16 variant runs
  int64_t ldx;
  int M, N, K;
  int kslice;         // K range per blockIdx.y
  int kc;             // K sub-slice staged per iteration
  int nseg;
  GemmSeg seg[MAX_SEG];
  float* P;           // [S, M, N]
};

// per-row data of a draft round
struct RowTab {
  int A, gamma;
  int anchor[MAX_ROWS];
  int pos[MAX_ROWS];  // block start position of each row
  int len[MAX_ROWS];  // context rows of each row
};

struct RopeCfg {
  double theta;
  int hd, nrot;       // rotated pairs: k < nrot turn, the rest pass through
};

struct EmbedArgs {
  const void* E; const void* Es; const void* Eb; int ekind; int group;
  const void* w_in; int act_bf16;
  int H; float eps; float scale; int mask_id;
  float* h; float* x;
  RowTab rows;
};

struct QkEpiArgs {
  const float* P; int S, M, N;
  const void* qn; const void* kn; int act_bf16;
  int nH, nKv, hd; float eps;
  RopeCfg rope;
  float* q;           // [A, nKv, nq, hd], nq = (nH/nKv)*gamma, row hl*gamma + g
  float* kb;          // [A, nKv, gamma, hd]
  float* vb;
  RowTab rows;
};

struct AttnRow {
  const void* k;      // [nKv, len, hd] act dtype
  const void* v;
};
struct AttnArgs {
  AttnRow row[MAX_ROWS];
  int len[MAX_ROWS];
  int split_off[MAX_ROWS + 1];  // prefix sum of key splits per row
  int A, gamma, nKv, nq, split;
  const float* q; const float* kb; const float* vb;
  float* opart;       // [nsplit, nKv, nq, hd] unnormalised
  float* ml;          // [nsplit, nKv, nq, 2] (running max, sum)
};

struct MergeArgs {
  int split_off[MAX_ROWS + 1];
  int A, gamma, nKv, nq, nH, hd;
  const float* opart; const float* ml;
  float* O;           // [A*gamma, nH*hd]
};

// row-wise epilogues over GEMM partials
struct RowEpiArgs {
  const float* P; int S, M, N;
  const void* w1; const void* w2; const void* scalar; int act_bf16;
  float eps;
  float* h;           // residual [M, N]
  float* x;           // next GEMM input [M, N]
  int mode;           // 0: o_proj (h += rms(o;w1); x = rms(h;w2))
                      // 1: down   (h = (h + rms(d;w1))*scalar; x = rms(h;w2))
                      // 2: plain  (x = rms(y;w1))
};

struct GateUpArgs {
  const float* P; int S, M, I;
  float* x;           // [M, I]
};

struct LmEpiArgs {
  const float* P; int S, M, V;
  float cap;          // <= 0: none
  const float* aux;   // [V] markov_w2 row norms, aux[V] = max markov_w1 row norm; null when rank 0
  float* z;           // [M, V]
  float* lo;          // [M, NC]
  float2* top;        // [M, NC, WALK_TOP] (value, index as float bits)
  int NC;
};

struct WalkArgs {
  RowTab rows;
  int V, NC, rank, wkind, group;
  const float* z; const float* lo; const float2* top;
  const void* w1; const void* w1s; const void* w1b;
  const void* w2; const void* w2s; const void* w2b;
  int32_t* tokens;
};

struct AuxArgs {
  int V, rank, wkind, group;
  const void* w1; const void* w1s; const void* w1b;
  const void* w2; const void* w2s; const void* w2b;
  float* aux;
};

struct KvEpiArgs {
  const float* P; int S, M, N;
  int B, L, layers, nKv, hd; float eps;
  const void* kn[16]; int act_bf16;
  RopeCfg rope;
  int pos0[MAX_ROWS];
  void* kout[16]; void* vout[16];
};

// launchers (return hipGetLastError())
hipError_t launch_gemm(const GemmArgs& a, int wkind, bool x_bf16, int mt, int S, hipStream_t st);
size_t gemm_lds_bytes(int wkind, bool x_bf16, int mt, int kc);
hipError_t launch_embed(const EmbedArgs& a, int M, hipStream_t st);
hipError_t launch_qk_epi(const QkEpiArgs& a, hipStream_t st);
hipError_t launch_attn(const AttnArgs& a, int hd, bool kv_bf16, int nsplit, hipStream_t st);
hipError_t launch_merge(const MergeArgs& a, hipStream_t st);
hipError_t launch_row_epi(const RowEpiArgs& a, hipStream_t st);
hipError_t launch_gateup(const GateUpArgs& a, hipStream_t st);
hipError_t launch_lm_epi(const LmEpiArgs& a, hipStream_t st);
hipError_t launch_walk(const WalkArgs& a, hipStream_t st);
hipError_t launch_aux(const AuxArgs& a, hipStream_t st);
hipError_t launch_kv_epi(const KvEpiArgs& a, hipStream_t st);

}  // namespace dsp
