// C ABI of the DSpark draft-round library: host-side validation, workspace
// planning and the kernel sequence of one round.  Every check runs before the
// first HIP call; the library never allocates device memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/dspark.h"
#include "dspark_kernels.hpp"

using namespace dsp;

namespace {

thread_local std::string g_err;

dspark_status fail(dspark_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

#define HIPCHECK(expr)                                                                  \
  do {                                                                                  \
    hipError_t e_ = (expr);                                                             \
    if (e_ != hipSuccess) return fail(DSPARK_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

struct Mat {
  int kind = -1;
  const void* w = nullptr;
  const void* s = nullptr;
  const void* b = nullptr;
  int64_t rows = 0, cols = 0;
};

struct LayerW {
  Mat q, k, o, g, u, d;
  const void *qn, *kn, *in, *pa, *pf, *pff, *scalar;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ---- optional launch timing -------------------------------------------------
struct ProfEntry {
  const char* name;
  hipEvent_t a, b;
};
bool g_prof = false;
std::vector<ProfEntry> g_prof_log;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t prof_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  // timing only: no system-scope fence at the record (no cache writeback
  // and invalidation between the timed kernels, which would slow the next
  // one and inflate the measured durations)
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

// run `launch` (returning hipError_t), bracketed by events when timing is on
template <class F>
hipError_t timed(const char* name, hipStream_t st, F&& launch) {
  if (!g_prof) return launch();
  ProfEntry e{name, prof_event(), prof_event()};
  // timing is best effort: a launch whose events cannot be recorded is not logged
  const bool ra = e.a && hipEventRecord(e.a, st) == hipSuccess;
  hipError_t r = launch();
  const bool rb = e.b && hipEventRecord(e.b, st) == hipSuccess;
  if (ra && rb) g_prof_log.push_back(e);
  return r;
}
int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

}  // namespace

struct dspark_model {
  dspark_config c;
  Mat embed, fc, lm, w1, w2, conf, wh;
  const void* conf_b = nullptr;
  const void* bh = nullptr;  // RNN head bias
  bool rnn = false;
  const void* hidden_norm = nullptr;
  const void* norm = nullptr;
  std::vector<LayerW> L;
  int nrot = 0;
  int nq = 0;
  int tall_rows = 48;  // GEMMs over at least this many rows take the tiled path (0: never)
};

namespace {

int act_bf16(const dspark_model* m) { return m->c.act_dtype == DSPARK_BF16 ? 1 : 0; }
int nc_of(const dspark_model* m) { return ceil_div(m->c.vocab_size, WALK_CHUNK); }

RopeCfg rope_of(const dspark_model* m) {
  RopeCfg r;
  r.step = std::pow((double)m->c.rope_theta, -2.0 / m->c.global_head_dim);
  r.hd = m->c.global_head_dim;
  r.nrot = m->nrot;
  return r;
}

// ---- GEMM planning --------------------------------------------------------
struct GemmPlan {
  int mt, kc, S, kslice, xmode;
  size_t pbytes;   // split-K partials
  size_t cwords;   // reduction counters
  int tall = TALL_NONE;  // tiled path over many rows: output tile
  int np = 0;            // tiled path: bf16 input planes (1: bf16 rows as they are; 2: hi + lo)
  size_t xbytes = 0;     // tiled path: the input planes (np == 2)
  size_t tbytes = 0;     // tiled path: partial products of a split K (S > 1)
};

GemmPlan plan_gemm_mt(int wk, int xmode, int M, int N, int K, int group_cols, int mt) {
  GemmPlan p;
  p.mt = mt;
  // sub-slice width: 256 (two sub-slices in flight)
  int kc = 256;
  while (kc > 128 && gemm_lds_bytes(wk, xmode, p.mt, kc) > 65536) kc /= 2;
  const int mblocks = ceil_div(M, 16 * p.mt);
  const int wgs = (N / 64) * mblocks;
  // Split K only while the grid is too small to give every CU a weight
  // stream; slices are multiples of 64, and normed inputs keep their norm
  // weights for the whole slice in LDS (at most 2048 wide).
  const int target = 256;
  int S = 1;
  if (wgs < target) S = std::min(16, ceil_div(target, wgs));
  if (xmode == XM_NORM) S = std::max(S, ceil_div(K, 2048));
  S = std::min(S, ceil_div(K, 64));
  // prefer the fully unrolled main loop (slices of 1, 2, 4 or 8 sub-slices
  // of 256): the fewest such slices that are at least S (K = 7680, S = 4:
  // 15 slices of 512 rather than 4 of 1920 on the generic loop)
  if (S > 1 && K % 256 == 0 && !(K % S == 0 && (K / S) % 256 == 0 && ((K / S / 256) & (K / S / 256 - 1)) == 0 &&
                                  K / S / 256 <= 8)) {
    for (int nch = 8; nch >= 1; nch /= 2)
      if ((K / 256) % nch == 0 && K / (256 * nch) >= S && K / (256 * nch) <= 32) {
        S = K / (256 * nch);
        break;
      }
  }
  const int kslice = ceil_div(ceil_div(K, S), 64) * 64;
  p.S = ceil_div(K, kslice);
  p.kslice = kslice;
  p.kc = std::min(kc, kslice);
  p.xmode = xmode;
  p.pbytes = p.S > 1 ? (size_t)p.S * mblocks * 16 * p.mt * N * 4 : 0;  // whole 16-row tiles
  p.cwords = gemm_counter_words(M, N, p.mt, group_cols);
  return p;
}

// One 16-row tile per workgroup, except the context projection over tall
// bf16 rows: 32-row tiles on eight-wave workgroups (two K halves) when the
// slice is a whole even number (2, 4 or 8) of 256-wide sub-slices, which
// reads each weight tile half as often as 16-row tiles.
GemmPlan plan_gemm(int wk, int xmode, int M, int N, int K, int group_cols, int tall_rows) {
  // many rows: the tiled path (bf16 weights; its epilogues need whole
  // 64-column blocks, head groups of at most 256 columns for the context
  // projection, and at most 256 statistics parts for normed inputs)
  // (the context projection, whose tiled epilogue reads the product in place
  // and so cannot split K, streams up to about 1024 rows: bf16 rows 23.6 us
  // against 38.2 us tiled at 512; hidden_norm(fc x) rows, the projection of
  // 64 / 256 target-feature rows 47.6 / 55.0 -> 38.3 / 51.1 us)
  const int64_t min_rows = group_cols > 0 ? std::max<int64_t>(4 * (int64_t)tall_rows, 1024) : tall_rows;
  if (wk == WK_BF16 && tall_rows > 0 && M >= min_rows && K % 64 == 0 && N % 64 == 0 &&
      (xmode != XM_NORM || K <= 256 * 64) && (group_cols == 0 || (group_cols <= 256 && N % group_cols == 0))) {
    GemmPlan p{};
    p.mt = 1;
    p.kc = 0;
    p.xmode = xmode;
    p.pbytes = 0;
    p.cwords = 0;
    // 128 x 128 tiles when they still give most CUs a tile, or when K is long
    // enough (>= 4096: the down projection) for split-K slices of >= 1024,
    // else 64 x 64 (their LDS reads per MFMA are twice as many);
    // fewer than 512 tiles split K (not the context projection, whose
    // epilogue reads the product in place) into slices of an even number of
    // 64-wide steps, for several workgroups per CU
    const int64_t tiles128 = (int64_t)ceil_div(M, 128) * ceil_div(N, 128);
    p.tall = (tiles128 >= 200 || (tiles128 >= 48 && K >= 4096)) ? TALL_128 : TALL_64;
    const int bt = p.tall == TALL_128 ? 128 : 64;
    const int64_t tiles = (int64_t)ceil_div(M, bt) * ceil_div(N, bt);
    const int steps = K / 64;
    int S = 1;
    if (tiles < 512 && group_cols == 0) S = (int)std::min<int64_t>(8, (768 + tiles - 1) / tiles);
    S = std::max(1, std::min(S, steps / 2));
    const int sl = 2 * ceil_div(ceil_div(steps, S), 2);  // steps per slice, even
    p.kslice = std::min(K, 64 * sl);
    p.S = ceil_div(K, p.kslice);
    p.np = xmode == XM_BF16 ? 1 : 2;
    p.xbytes = p.np == 2 ? (size_t)2 * M * K * 2 : 0;
    p.tbytes = p.S > 1 ? (size_t)p.S * M * N * 4 : 0;
    return p;
  }
  if (group_cols > 0 && wk == WK_BF16 && xmode == XM_BF16 && M >= 32) {
    const GemmPlan p2 = plan_gemm_mt(wk, xmode, M, N, K, group_cols, 2);
    const int nch = p2.kslice / 256;
    if (p2.kc == 256 && K % p2.kslice == 0 && p2.kslice % 256 == 0 && p2.S == 1 && (nch == 2 || nch == 4 || nch == 8))
      return p2;
  }
  return plan_gemm_mt(wk, xmode, M, N, K, group_cols, 1);
}

// workspace of the tiled path: bf16 input planes, and the product of the
// GEMMs whose epilogue output is not the product itself (q|k, gate|up)
struct TallBufs {
  uint16_t* xop = nullptr;
  float* T = nullptr;
};

// a weight-streaming context projection that leaves its K/V epilogue to a
// separate launch (no split K, head groups k_kv_epi takes): it needs no
// reduction counters
bool kv_deferred(const GemmPlan& p) { return p.tall == TALL_NONE && p.S == 1; }

// gate|up whose tiles form gelu_tanh(gate) * up themselves (tiled path)
bool fused_gelu(const GemmPlan& p, int64_t N) { return p.tall == TALL_128 && p.S == 1 && p.np == 2 && N % 128 == 0; }

// x_planes: the tiled path's input planes are already in tb.xop (the
// attention merge or the fused gate|up wrote them), so no input preparation runs
// next: on the tiled path, a split-K EPI_SUMS epilogue that also forms the
// next GEMM's input planes (k_sums_prep) instead of the product's row
// statistics (its T, S, M and K are filled in here)
hipError_t run_gemm(const GemmPlan& p, GemmArgs a, const EpiArgs& e, int epi, int wk, hipStream_t st,
                    const TallBufs& tb = TallBufs{}, bool x_planes = false, const SumsPrepArgs* next = nullptr) {
  a.kslice = p.kslice;
  a.kc = p.kc;
  if (p.tall == TALL_NONE && epi == EPI_KV && kv_deferred(p)) {
    // the context projection without split K: product to Y, then the
    // norms and RoPE in their own launch
    EpiArgs ed = e;
    ed.kv_defer = 1;
    const hipError_t r = launch_gemm(a, ed, epi, wk, p.xmode, p.mt, p.S, st);
    if (r != hipSuccess) return r;
    return launch_gemm_epi(a, ed, EPI_KV, nullptr, 0, 1, 0, st);
  }
  if (p.tall == TALL_NONE) return launch_gemm(a, e, epi, wk, p.xmode, p.mt, p.S, st);
  TallArgs t{};
  if (p.xmode == XM_BF16) {
    t.X = (const uint16_t*)a.X;
    t.ldx = a.ldx;
    t.plane = 0;
  } else {
    if (!tb.xop) return hipErrorInvalidValue;
    if (!x_planes) {
      const hipError_t r = launch_xprep(a, p.xmode, tb.xop, (int64_t)a.M * a.K, st);
      if (r != hipSuccess) return r;
    }
    t.X = tb.xop;
    t.ldx = a.K;
    t.plane = (int64_t)a.M * a.K;
  }
  t.M = a.M;
  t.N = a.N;
  t.K = a.K;
  t.kslice = p.kslice;
  t.nseg = a.nseg;
  for (int i = 0; i < MAX_SEG; ++i) t.seg[i] = a.seg[i];
  // the product goes where the epilogue's own output goes when the epilogue
  // only reads it back in place (row statistics, softcap) or reads it from
  // there (context K/V); q|k and gate|up, and the partial products of a
  // split K, take the separate buffer
  t.tstride = 0;
  if (p.S > 1) {
    if (!tb.T || epi == EPI_KV) return hipErrorInvalidValue;
    t.T = tb.T;
    t.ldt = a.N;
    t.tstride = (int64_t)a.M * a.N;
  } else if (epi == EPI_SUMS) {
    t.T = e.Y;
    t.ldt = e.ldy;
  } else if (epi == EPI_KV || epi == EPI_LM) {
    t.T = e.Y;
    t.ldt = a.N;
  } else {
    if (!tb.T) return hipErrorInvalidValue;
    t.T = tb.T;
    t.ldt = a.N;
  }
  // logits: softcap and the walk's chunk bounds in the tiled kernel itself
  // when its 128 x 128 tiles hold the final product (not when sampling: the
  // noise is added by the separate logits epilogue, which keeps the tiled
  // kernel's store loop free of it)
  if (epi == EPI_LM && p.tall == TALL_128 && p.S == 1 && a.N % 64 == 0 && !(e.smp.temperature > 0.f)) {
    t.lm = 1;
    t.cap = e.cap;
    t.aux = e.aux;
    t.lohi = e.lohi;
    t.NC = e.NC;
    return launch_tall(t, p.tall, p.np, p.S, st);
  }
  // gate|up: gelu_tanh(gate) * up in the tiled kernel itself when its
  // 128 x 128 tiles hold the final product of hi + lo planes
  if (epi == EPI_GELU && fused_gelu(p, a.N)) {
    t.gelu = 1;
    t.act = e.act;
    t.ld_act = e.ld_act;
    t.act_planes = e.act_planes;
    t.act_plane = e.act_plane;
    return launch_tall(t, p.tall, p.np, p.S, st);
  }
  hipError_t r = launch_tall(t, p.tall, p.np, p.S, st);
  if (r != hipSuccess) return r;
  if (epi == EPI_SUMS && next) {
    SumsPrepArgs sp = *next;
    sp.T = t.T;
    sp.ldt = t.ldt;
    sp.tstride = t.tstride;
    sp.S = p.S;
    sp.M = a.M;
    sp.K = a.N;
    return launch_sums_prep(sp, st);
  }
  return launch_gemm_epi(a, e, epi, t.T, t.ldt, p.S, t.tstride, st);
}

GemmSeg seg_of(const Mat& w, int n0) {
  GemmSeg s;
  s.w = w.w;
  s.s = w.s;
  s.b = w.b;
  s.n0 = n0;
  s.pad_ = 0;
  return s;
}

// ---- draft workspace layout ---------------------------------------------
// Row pitches of the fp32 activation buffers are padded by 64 floats so that
// the rows of one column range fall on different L2 / HBM channels.
constexpr int ROW_PAD = 64;

struct DraftLayout {
  size_t hA, hB, Y, sums, rt, scal, O, act, P, cnt, q, kb, vb, ssq, opart, ml, z, lohi, xop, xop2, T, conf, total;
  bool dn_planes;  // the fused gate|up writes the tiled down projection's input planes (xop2)
  int64_t ldh, ldo, ldact;
  GemmPlan qk, o, gu, dn, lm;
  size_t cwords;
  int nsplit_max;
};

// context keys per attention split: a multiple of the 32-key staging chunk,
// grown with the total context so that at most ~512 context splits exist
int attn_split(int64_t total_ctx) {
  int64_t s = (total_ctx + 511) / 512;
  s = (s + ATT_KEYS - 1) / ATT_KEYS * ATT_KEYS;
  return (int)std::max<int64_t>(ATT_KEYS, s);
}

// the same for the wide kernel (every query row of a kv head per
// workgroup, one workgroup per compute unit): the context splits and the A
// block splits fit the 256 compute units of an MI355X in one round (each row
// adds up to one short tail split), so no second round runs at part
// occupancy, and fewer partial outputs are merged
constexpr int ATTN_CUS = 256;
int attn_split_wide(int64_t total_ctx, int A) {
  const int64_t slots = std::max<int64_t>(ATTN_CUS - 2 * (int64_t)A, ATTN_CUS / 2);
  int64_t s = (total_ctx + slots - 1) / slots;
  s = (s + ATT_KEYS - 1) / ATT_KEYS * ATT_KEYS;
  return (int)std::max<int64_t>(ATT_KEYS, s);
}
// contexts long enough in total for the wide attention kernel
constexpr int64_t ATTN_WIDE_MIN_KEYS = 2048;

// Attention splits of a round over A rows whose contexts hold total_ctx keys:
// each row has ceil(L_a / split) context splits and one block split, with
// split >= ATT_KEYS and split >= total_ctx / 512 (attn_split; the wide plan's
// splits are longer still), so sum_a ceil(L_a / split) < total_ctx / split + A
// and there are at most min(512, ceil(total_ctx / ATT_KEYS)) + 2A of them.
int64_t nsplit_bound(int64_t total_ctx, int A) {
  return std::min<int64_t>(512, (total_ctx + ATT_KEYS - 1) / ATT_KEYS) + 2 * (int64_t)A;
}

DraftLayout draft_layout(const dspark_model* m, int A, bool with_z, int64_t total_ctx) {
  const dspark_config& c = m->c;
  const int M = A * c.block_size, H = c.hidden_size, I = c.intermediate_size, hd = c.global_head_dim;
  const int nH = c.num_attention_heads, nKv = c.num_global_key_value_heads;
  const int wk = c.weight_dtype;
  DraftLayout d;
  const int tr = m->tall_rows;
  // gate|up gains from the tiled path earlier: from two thirds of the
  // threshold (32 rows by default; measured over two blocks of 16 rows:
  // gate|up 31.9 -> 27.5 us per launch with its input and epilogue launches,
  // while q|k, o, down and lm_head stay ahead on the streaming kernel)
  const int tr_wide = tr > 0 ? std::max(1, 2 * tr / 3) : 0;
  d.qk = plan_gemm(wk, XM_NORM, M, (nH + nKv) * hd, H, 0, tr);
  d.o = plan_gemm(wk, XM_F32, M, H, nH * hd, 0, tr);
  d.gu = plan_gemm(wk, XM_NORM, M, 2 * I, H, 0, tr_wide);
  d.dn = plan_gemm(wk, XM_F32, M, H, I, 0, tr);
  d.lm = plan_gemm(wk, XM_NORM, M, c.vocab_size, H, 0, tr);
  // the logits feed no attention, so on the fused tiled path lm_head
  // multiplies the hi plane alone (bf16-rounded final hidden rows): half the
  // MFMAs, a third fewer LDS reads
  if (d.lm.tall == TALL_128 && d.lm.S == 1 && d.lm.np == 2 && c.vocab_size % 64 == 0) d.lm.np = 1;
  const size_t pmax = std::max({d.qk.pbytes, d.o.pbytes, d.gu.pbytes, d.dn.pbytes, d.lm.pbytes, (size_t)4});
  d.cwords = std::max({d.qk.cwords, d.o.cwords, d.gu.cwords, d.dn.cwords, d.lm.cwords});
  d.nsplit_max = (int)nsplit_bound(total_ctx, A);
  const int NC = nc_of(m);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  d.ldh = H + ROW_PAD;
  d.ldo = (int64_t)nH * hd + ROW_PAD;
  d.ldact = I + ROW_PAD;
  d.hA = take((size_t)M * d.ldh * 4);
  d.hB = take((size_t)M * d.ldh * 4);
  d.Y = take((size_t)M * d.ldh * 4);
  d.sums = take((size_t)(H / 64) * M * sizeof(RowStats));
  d.rt = take((size_t)M * (hd / 2) * 8);
  d.scal = take((size_t)(c.num_hidden_layers + 1) * 4);
  d.O = take((size_t)M * d.ldo * 4);
  d.act = take((size_t)M * d.ldact * 4);
  d.P = take(pmax);
  d.cnt = take(d.cwords * 4);
  d.q = take((size_t)A * nKv * m->nq * hd * 4);
  d.kb = take((size_t)A * nKv * c.block_size * hd * 4);
  d.vb = take((size_t)A * nKv * c.block_size * hd * 4);
  d.ssq = take((size_t)(nH + nKv) * (hd / 64) * M * 4);
  // fp32 partials [split, kvh, nq, hd] (fp32 cache), or fp16 ones in groups
  // of 16 query rows (bf16 cache)
  const size_t part_bytes = c.act_dtype == DSPARK_BF16 ? (size_t)((m->nq + 15) / 16) * 16 * hd * 2
                                                       : (size_t)m->nq * hd * 4;
  d.opart = take((size_t)d.nsplit_max * nKv * part_bytes);
  d.ml = take((size_t)d.nsplit_max * nKv * m->nq * 2 * 4);
  d.z = with_z ? take((size_t)M * c.vocab_size * 4) : 0;
  d.lohi = take((size_t)M * NC * 8);
  d.xop = take(std::max({d.qk.xbytes, d.o.xbytes, d.gu.xbytes, d.dn.xbytes, d.lm.xbytes, (size_t)4}));
  d.dn_planes = fused_gelu(d.gu, 2 * (int64_t)I) && d.dn.tall != TALL_NONE && d.dn.np == 2;
  d.xop2 = take(d.dn_planes ? (size_t)2 * M * I * 2 : 4);
  d.T = take(std::max({d.qk.tall ? (size_t)M * (nH + nKv) * hd * 4 : 0, d.gu.tall ? (size_t)M * 2 * I * 4 : 0,
                       d.qk.tbytes, d.o.tbytes, d.gu.tbytes, d.dn.tbytes, d.lm.tbytes, (size_t)4}));
  d.conf = take((size_t)M * 4);
  d.total = off;
  return d;
}

// ---- projection workspace layout -----------------------------------------
struct ProjLayout {
  size_t P, Y, C, sums, cnt, xop, T, total;
  GemmPlan fc, kp;
  size_t cwords;
  int lay_per_gemm;
};

int xmode_in(const dspark_model* m) { return m->c.act_dtype == DSPARK_BF16 ? XM_BF16 : XM_F32; }

ProjLayout proj_layout(const dspark_model* m, int input_kind, int B, int L) {
  const dspark_config& c = m->c;
  const int M = B * L, H = c.hidden_size, hd = c.global_head_dim, nKv = c.num_global_key_value_heads;
  ProjLayout p{};
  p.lay_per_gemm = std::min(c.num_hidden_layers, MAX_SEG);
  const int Nk = p.lay_per_gemm * nKv * hd;
  const bool feats = input_kind == DSPARK_INPUT_TARGET_FEATURES;
  size_t pbytes = 4;
  if (feats) {
    p.fc = plan_gemm(c.weight_dtype, xmode_in(m), M, H, c.fc_in, 0, m->tall_rows);
    pbytes = std::max(pbytes, p.fc.pbytes);
    p.cwords = p.fc.cwords;
  }
  p.kp = plan_gemm(c.weight_dtype, feats ? XM_NORM : xmode_in(m), M, Nk, H, hd, m->tall_rows);
  size_t xbytes = std::max(p.fc.xbytes, p.kp.xbytes);
  const size_t tbytes = p.fc.tbytes;  // (the context projection never splits K on the tiled path)
  pbytes = std::max(pbytes, p.kp.pbytes);
  p.cwords = std::max(p.cwords, p.kp.cwords);
  // a last, smaller group of layers is planned on its own (it may split K)
  const int rem = c.num_hidden_layers % p.lay_per_gemm;
  if (rem) {
    const GemmPlan r = plan_gemm(c.weight_dtype, p.kp.xmode, M, rem * nKv * hd, H, hd, m->tall_rows);
    pbytes = std::max(pbytes, r.pbytes);
    xbytes = std::max(xbytes, r.xbytes);
    p.cwords = std::max(p.cwords, r.cwords);
  }
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  p.P = take(pbytes);
  p.Y = take((size_t)M * Nk * 4);
  p.C = feats ? take((size_t)M * H * 4) : 0;
  p.sums = feats ? take((size_t)(H / 64) * M * sizeof(RowStats)) : 0;
  p.cnt = take(p.cwords * 4);
  p.xop = take(std::max(xbytes, (size_t)4));
  p.T = take(std::max(tbytes, (size_t)4));
  p.total = off;
  return p;
}

// ---- model creation --------------------------------------------------------
dspark_status check_shapes(const dspark_config& c) {
  if (!c.attention_k_eq_v)
    return fail(DSPARK_ERR_UNSUPPORTED, "attention_k_eq_v=false needs a v_proj path; only V == K is implemented");
  if (c.markov_rank > 0 && !c.markov_head_vanilla && !c.markov_head_rnn)
    return fail(DSPARK_ERR_UNSUPPORTED, "only the vanilla and rnn Markov heads are implemented");
  if (c.markov_head_vanilla && c.markov_head_rnn)
    return fail(DSPARK_ERR_INVALID_ARG, "markov_head_vanilla and markov_head_rnn both set");
  if (!c.activation_gelu_tanh)
    return fail(DSPARK_ERR_UNSUPPORTED, "only the gelu_pytorch_tanh activation is implemented");
  if (c.hidden_size <= 0 || c.num_hidden_layers <= 0 || c.num_attention_heads <= 0 || c.global_head_dim <= 0 ||
      c.num_global_key_value_heads <= 0 || c.intermediate_size <= 0 || c.vocab_size <= 0 || c.block_size <= 0 ||
      c.markov_rank < 0 || c.fc_in < 0)
    return fail(DSPARK_ERR_INVALID_ARG, "config sizes must be positive");
  if (c.num_attention_heads % c.num_global_key_value_heads)
    return fail(DSPARK_ERR_SHAPE, "num_attention_heads %% num_global_key_value_heads != 0");
  if (c.global_head_dim != 64 && c.global_head_dim != 128 && c.global_head_dim != 256)
    return fail(DSPARK_ERR_UNSUPPORTED, "global_head_dim %d not built (64, 128, 256)", c.global_head_dim);
  if (c.hidden_size % 64 || c.intermediate_size % 64 || c.fc_in % 64)
    return fail(DSPARK_ERR_UNSUPPORTED, "hidden, intermediate and fc input sizes must be multiples of 64");
  if (c.hidden_size > 8192 || c.intermediate_size > (1 << 20))
    return fail(DSPARK_ERR_UNSUPPORTED, "hidden_size > 8192 not built");
  if (c.num_hidden_layers > MAX_LAYERS) return fail(DSPARK_ERR_UNSUPPORTED, "more than %d layers not built", MAX_LAYERS);
  // the walk packs (step, chunk) into one word with 24 bits for the chunk;
  // 2^22 keeps every vocabulary product in int32 range as well
  if (c.vocab_size % 64 || c.vocab_size > (1 << 22))
    return fail(DSPARK_ERR_UNSUPPORTED, "vocab_size must be a multiple of 64 and at most %d", 1 << 22);
  if (c.block_size > 32) return fail(DSPARK_ERR_UNSUPPORTED, "block_size > 32 not built");
  if ((c.num_attention_heads / c.num_global_key_value_heads) * c.block_size > 128)
    return fail(DSPARK_ERR_UNSUPPORTED, "more than 128 query rows per kv head not built");
  if (c.markov_rank > 256 || c.markov_rank % 8)
    return fail(DSPARK_ERR_UNSUPPORTED, "markov_rank must be a multiple of 8 and at most 256");
  if (c.mask_token_id < 0 || c.mask_token_id >= c.vocab_size)
    return fail(DSPARK_ERR_INVALID_ARG, "mask_token_id out of range");
  if (c.enable_confidence_head && c.confidence_head_with_markov && c.markov_rank == 0)
    return fail(DSPARK_ERR_INVALID_ARG, "confidence_head_with_markov requires markov_rank > 0");
  if (c.block_size > CONF_MAX_GAMMA) return fail(DSPARK_ERR_UNSUPPORTED, "block_size > %d not built", CONF_MAX_GAMMA);
  if (!(c.rope_theta > 0) || !(c.partial_rotary_factor >= 0 && c.partial_rotary_factor <= 1) || !(c.rms_norm_eps >= 0))
    return fail(DSPARK_ERR_INVALID_ARG, "rope_theta, partial_rotary_factor or rms_norm_eps out of range");
  if (c.act_dtype != DSPARK_F32 && c.act_dtype != DSPARK_BF16)
    return fail(DSPARK_ERR_UNSUPPORTED, "act_dtype must be F32 or BF16");
  if (c.weight_dtype != DSPARK_F32 && c.weight_dtype != DSPARK_BF16 && c.weight_dtype != DSPARK_Q4)
    return fail(DSPARK_ERR_UNSUPPORTED, "weight_dtype must be F32, BF16 or Q4");
  if (c.weight_dtype == DSPARK_Q4) {
    if (c.group_size != 64) return fail(DSPARK_ERR_UNSUPPORTED, "Q4 group size %d not built (64)", c.group_size);
    if (c.markov_rank % 64) return fail(DSPARK_ERR_UNSUPPORTED, "Q4 Markov tables need rank %% 64 == 0");
  }
  return DSPARK_OK;
}

dspark_status check_config(const dspark_config& c) {
  const dspark_status st = check_shapes(c);
  if (st) return st;
  // The first GPU run of a 4-bit round faulted and no cause has been shown
  // yet; the path stays switched off until one is.
  if (c.weight_dtype == DSPARK_Q4)
    return fail(DSPARK_ERR_UNSUPPORTED, "4-bit weights are disabled in this library version (an unexplained GPU fault)");
  return DSPARK_OK;
}

// ---- fixed scratch for callers that cannot allocate ------------------------
// The workspace of dspark_draft_rows_noalloc: one array per GPU in the
// library's own code object (each GPU the library runs on holds it until the
// process ends).  In host code `scratch` is only a host-side stand-in; its
// device address is looked up once per device (hipGetSymbolAddress, with that
// device current) and only that address is ever handed to kernels.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[NOALLOC_MAX_DEVICES] = {};

// the device address of the current device's scratch array
dspark_status scratch_address(void** out) {
  int dev = -1;
  HIPCHECK(hipGetDevice(&dev));
  if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return fail(DSPARK_ERR_UNSUPPORTED, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    HIPCHECK(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
    if (!ptr || ((uintptr_t)ptr & 255)) return fail(DSPARK_ERR_HIP, "scratch array has no usable device address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DSPARK_OK;
}

}  // namespace

extern "C" {

const char* dspark_last_error(void) { return g_err.c_str(); }

dspark_status dspark_stream_block_of(int gx, int S, int R, int x, int y, int z, int* bx, int* by, int* bz) {
  g_err.clear();
  if (gx <= 0 || S <= 0 || R <= 0 || x < 0 || x >= gx || y < 0 || y >= S || z < 0 || z >= R || !bx || !by || !bz)
    return fail(DSPARK_ERR_INVALID_ARG, "stream_block_of: bad grid or workgroup");
  dsp::stream_block_of(gx, S, R, x, y, z, *bx, *by, *bz);
  return DSPARK_OK;
}

dspark_status dspark_tall_tile_of(int gx, int gy, int w, int* bx, int* by) {
  g_err.clear();
  if (gx <= 0 || gy <= 0 || !bx || !by || w < 0 || (int64_t)w >= (int64_t)gx * gy)
    return fail(DSPARK_ERR_INVALID_ARG, "grid %d x %d, workgroup %d", gx, gy, w);
  tall_tile_of(gx, gy, w, *bx, *by);
  return DSPARK_OK;
}

// ---- host replay of the 4-bit weight addresses ------------------------------
// Every address that the 4-bit branches of the kernels form, evaluated on the
// host with the kernels' own index functions (q4_word, q4_group,
// q4_gemm_word, q4_gemm_group, wave_col, xsum_offset, xbuf_bytes) over the
// launch plans the library makes, each checked against the buffer it reads.
extern "C++" {
namespace {
struct Q4Replay {
  int64_t n = 0;
  dspark_status st = DSPARK_OK;
};

// k_gemm's weight loads and per-group activation sums: the only GEMM variant
// built for 4-bit weights is the streaming one with one 16-row tile and four
// waves per workgroup, sub-slices of kc (KCMAX 256, SMAX = 8 steps of 32)
template <int EPI>
void q4_replay_gemm(Q4Replay& r, const char* role, const GemmPlan& p, int N, int K, int hd, int nseg,
                    const int64_t* seg_rows, const int* seg_n0) {
  if (r.st) return;
  constexpr int KCMAX = 256, SMAX = KCMAX / 32;
  if (p.tall != TALL_NONE || p.mt != 1 || p.kc > KCMAX || p.kc % 64 || p.kslice % 64 || K % 64 || N % 64) {
    r.st = fail(DSPARK_ERR_SHAPE, "%s: plan tall %d mt %d kc %d kslice %d K %d N %d outside the 4-bit GEMM's domain",
                role, p.tall, p.mt, p.kc, p.kslice, K, N);
    return;
  }
  const int KC = p.kc, ngmax = KC >> 6;
  // the sums sit after the activation planes and inside one staging buffer;
  // a 16-row tile double-buffers within the launch's dynamic LDS
  if (xsum_offset(p.xmode, 1, KC) + (size_t)16 * ngmax * 4 > xbuf_bytes(WK_Q4, p.xmode, 1, KC) ||
      2 * xbuf_bytes(WK_Q4, p.xmode, 1, KC) > gemm_lds_bytes(WK_Q4, p.xmode, 1, KC) ||
      gemm_lds_bytes(WK_Q4, p.xmode, 1, KC) > 65536) {
    r.st = fail(DSPARK_ERR_SHAPE, "%s: 4-bit staging buffers exceed the launch's LDS", role);
    return;
  }
  // how often each word and each scale of every segment is read by one row
  // block of the grid: every word once, every scale once per lane group
  std::vector<std::vector<uint8_t>> wcount(nseg), gcount(nseg);
  for (int i = 0; i < nseg; ++i) {
    wcount[i].assign((size_t)(seg_rows[i] * (K >> 3)), 0);
    gcount[i].assign((size_t)(seg_rows[i] * (K / 64)), 0);
  }
  for (int cb = 0; cb < N / 64; ++cb)
    for (int w = 0; w < 4; ++w) {
      const int n0w = wave_col<EPI>(cb, w, N, hd);
      int si = 0;
      for (int i = 1; i < nseg; ++i)
        if (n0w >= seg_n0[i]) si = i;
      const int64_t rows = seg_rows[si];
      const int64_t words = rows * (K >> 3), groups = rows * (K / 64);
      for (int col = 0; col < 16; ++col) {
        const int64_t wrow = (int64_t)(n0w - seg_n0[si] + col);
        if (wrow < 0 || wrow >= rows) {
          r.st = fail(DSPARK_ERR_SHAPE, "%s: column block %d wave %d reads weight row %lld of %lld", role, cb, w,
                      (long long)wrow, (long long)rows);
          return;
        }
        for (int y = 0; y < p.S; ++y) {
          const int kbeg = y * p.kslice, kend = std::min(K, kbeg + p.kslice);
          for (int kc = kbeg; kc < kend; kc += KC) {
            const int len = std::min(KC, kend - kc), nsteps = len >> 5;
            if (len % 64) {
              r.st = fail(DSPARK_ERR_SHAPE, "%s: sub-slice of %d codes (not whole 64-groups)", role, len);
              return;
            }
            for (int gq = 0; gq < 4; ++gq)
              for (int j = 0; j < SMAX / 2; ++j) {
                if (2 * j >= nsteps) continue;
                const int64_t wd = q4_gemm_word(wrow, K, kc, gq, j), gi = q4_gemm_group(wrow, K, kc, j);
                // both words hold codes of this row inside the sub-slice
                const int64_t k0 = (wd - wrow * (K >> 3)) * 8;
                r.n += 3;
                if (wd < 0 || wd + 1 >= words || k0 < kc || k0 + 16 > kc + len || gi < 0 || gi >= groups ||
                    gi - wrow * (K / 64) != (kc + 64 * j) / 64) {
                  r.st = fail(DSPARK_ERR_SHAPE, "%s: row %lld k %d lane group %d group %d: word %lld of %lld, "
                              "scale %lld of %lld", role, (long long)wrow, kc, gq, j, (long long)wd,
                              (long long)words, (long long)gi, (long long)groups);
                  return;
                }
                wcount[si][wd] += 1;
                wcount[si][wd + 1] += 1;
                gcount[si][gi] += 1;
              }
            // the staging's group sums: row ml < 16, group of the 8-code piece k8
            for (int k8 = 0; k8 < (len >> 3); ++k8) {
              const int idx = 15 * ngmax + (k8 >> 3);
              ++r.n;
              if ((k8 >> 3) >= ngmax || idx >= 16 * ngmax) {
                r.st = fail(DSPARK_ERR_SHAPE, "%s: group sum %d of %d", role, idx, 16 * ngmax);
                return;
              }
            }
          }
        }
      }
    }
  for (int i = 0; i < nseg; ++i) {
    for (size_t x = 0; x < wcount[i].size(); ++x)
      if (wcount[i][x] != 1) {
        r.st = fail(DSPARK_ERR_SHAPE, "%s: segment %d word %zu read %d times by one row block", role, i, x,
                    (int)wcount[i][x]);
        return;
      }
    for (size_t x = 0; x < gcount[i].size(); ++x)
      if (gcount[i][x] != 4) {
        r.st = fail(DSPARK_ERR_SHAPE, "%s: segment %d scale %zu read %d times by one row block", role, i, x,
                    (int)gcount[i][x]);
        return;
      }
  }
}

// element reads of a 4-bit table (embedding, Markov tables, the RNN matrix,
// the confidence projection): rows [r0, r1) and every column
void q4_replay_table(Q4Replay& r, const char* role, int64_t rows, int cols, int group, int64_t r0, int64_t r1) {
  if (r.st) return;
  const int64_t words = rows * (cols >> 3), groups = rows * (cols / group);
  for (int64_t row = r0; row < r1; ++row)
    for (int k = 0; k < cols; ++k) {
      const int64_t wd = q4_word(row, cols, k), gi = q4_group(row, cols, group, k);
      ++r.n;
      if (row < 0 || row >= rows || wd < 0 || wd >= words || gi < 0 || gi >= groups) {
        r.st = fail(DSPARK_ERR_SHAPE, "%s: element (%lld, %d): word %lld of %lld, scale %lld of %lld", role,
                    (long long)row, k, (long long)wd, (long long)words, (long long)gi, (long long)groups);
        return;
      }
    }
}
}  // namespace
}  // extern "C++"

dspark_status dspark_q4_address_check(const dspark_config* cfg, int A, const int32_t* anchors_host, int64_t ctx_rows,
                                      int input_kind, int64_t* n_checked) {
  g_err.clear();
  if (!cfg || !anchors_host || A <= 0 || A > MAX_ROWS || ctx_rows <= 0 || ctx_rows > (1 << 24))
    return fail(DSPARK_ERR_INVALID_ARG, "null config or anchors, or A / ctx_rows out of range");
  const dspark_config& c = *cfg;
  if (c.weight_dtype != DSPARK_Q4) return fail(DSPARK_ERR_INVALID_ARG, "not a 4-bit config");
  dspark_status st = check_shapes(c);
  if (st) return st;
  if (input_kind == DSPARK_INPUT_TARGET_FEATURES && c.fc_in == 0)
    return fail(DSPARK_ERR_UNSUPPORTED, "model has no fc / hidden_norm");
  for (int a = 0; a < A; ++a)
    if (anchors_host[a] < 0 || anchors_host[a] >= c.vocab_size)
      return fail(DSPARK_ERR_INVALID_ARG, "anchor %d out of range", a);
  // a model with the config's sizes and no tensors: the layouts read sizes only
  dspark_model m;
  m.c = c;
  const int rotated = (int)std::floor(c.global_head_dim * c.partial_rotary_factor);
  m.nrot = std::min((rotated + 1) / 2, c.global_head_dim / 2);
  m.nq = (c.num_attention_heads / c.num_global_key_value_heads) * c.block_size;
  const int H = c.hidden_size, I = c.intermediate_size, hd = c.global_head_dim, V = c.vocab_size;
  const int nH = c.num_attention_heads, nKv = c.num_global_key_value_heads, G = c.group_size, r = c.markov_rank;
  Q4Replay rp;
  // the round's GEMMs (weights [out, in]; segments as the round passes them)
  const DraftLayout d = draft_layout(&m, A, true, 1);
  {
    const int64_t rows[2] = {(int64_t)nH * hd, (int64_t)nKv * hd};
    const int n0[2] = {0, nH * hd};
    q4_replay_gemm<EPI_QK>(rp, "q|k", d.qk, (nH + nKv) * hd, H, hd, 2, rows, n0);
  }
  {
    const int64_t rows[1] = {H};
    const int n0[1] = {0};
    q4_replay_gemm<EPI_SUMS>(rp, "o", d.o, H, nH * hd, hd, 1, rows, n0);
    q4_replay_gemm<EPI_SUMS>(rp, "down", d.dn, H, I, hd, 1, rows, n0);
  }
  {
    const int64_t rows[2] = {I, I};
    const int n0[2] = {0, I};
    q4_replay_gemm<EPI_GELU>(rp, "gate|up", d.gu, 2 * I, H, hd, 2, rows, n0);
  }
  {
    const int64_t rows[1] = {V};
    const int n0[1] = {0};
    q4_replay_gemm<EPI_LM>(rp, "lm_head", d.lm, V, H, hd, 1, rows, n0);
  }
  // the context projection: fc, then k_proj over groups of layers
  const ProjLayout pl = proj_layout(&m, input_kind, 1, (int)ctx_rows);
  if (input_kind == DSPARK_INPUT_TARGET_FEATURES) {
    const int64_t rows[1] = {H};
    const int n0[1] = {0};
    q4_replay_gemm<EPI_SUMS>(rp, "fc", pl.fc, H, c.fc_in, hd, 1, rows, n0);
  }
  for (int l0 = 0; l0 < c.num_hidden_layers; l0 += pl.lay_per_gemm) {
    const int nl = std::min(pl.lay_per_gemm, c.num_hidden_layers - l0);
    const GemmPlan gp = nl == pl.lay_per_gemm ? pl.kp
                                              : plan_gemm(c.weight_dtype, pl.kp.xmode, (int)ctx_rows, nl * nKv * hd, H,
                                                          hd, m.tall_rows);
    int64_t rows[MAX_SEG];
    int n0[MAX_SEG];
    for (int i = 0; i < nl; ++i) {
      rows[i] = (int64_t)nKv * hd;
      n0[i] = i * nKv * hd;
    }
    q4_replay_gemm<EPI_KV>(rp, "k_proj", gp, nl * nKv * hd, H, hd, nl, rows, n0);
  }
  // element reads: the embedding rows of the anchors and the mask id, the
  // Markov tables (walk bound over every row, walk and confidence over any
  // previous token), the RNN matrix, the confidence projection
  for (int a = 0; a < A; ++a) q4_replay_table(rp, "embed", V, H, G, anchors_host[a], anchors_host[a] + 1);
  q4_replay_table(rp, "embed", V, H, G, c.mask_token_id, c.mask_token_id + 1);
  if (r > 0) {
    q4_replay_table(rp, "markov_w1", V, r, G, 0, V);
    q4_replay_table(rp, "markov_w2", V, r, G, 0, V);
    if (c.markov_head_rnn) q4_replay_table(rp, "rnn_wh", r, r, G, 0, r);
  }
  if (c.enable_confidence_head)
    q4_replay_table(rp, "confidence proj", 1, H + (c.confidence_head_with_markov ? r : 0), G, 0, 1);
  if (n_checked) *n_checked = rp.n;
  return rp.st;
}

void dspark_profile_enable(int on) { g_prof = on != 0; }

int dspark_profile_read(dspark_kernel_time* out, int max) {
  std::vector<dspark_kernel_time> acc;
  for (const ProfEntry& e : g_prof_log) {
    float ms = 0.f;
    if (hipEventSynchronize(e.b) != hipSuccess || hipEventElapsedTime(&ms, e.a, e.b) != hipSuccess) ms = 0.f;
    size_t i = 0;
    while (i < acc.size() && std::strcmp(acc[i].name, e.name) != 0) ++i;
    if (i == acc.size()) acc.push_back(dspark_kernel_time{e.name, 0, 0.0});
    acc[i].launches += 1;
    acc[i].ms += ms;
    g_event_pool.push_back(e.a);
    g_event_pool.push_back(e.b);
  }
  g_prof_log.clear();
  int n = 0;
  for (; n < (int)acc.size() && n < max; ++n)
    if (out) out[n] = acc[n];
  return n;
}

dspark_status dspark_model_create(const dspark_config* cfg, const dspark_weight* table, int n, dspark_model** out) {
  g_err.clear();
  if (!cfg || !table || !out || n <= 0) return fail(DSPARK_ERR_INVALID_ARG, "null config, table or output");
  *out = nullptr;
  dspark_status st = check_config(*cfg);
  if (st) return st;
  const dspark_config& c = *cfg;
  std::map<std::string, const dspark_weight*> byname;
  for (int i = 0; i < n; ++i) {
    if (!table[i].name) return fail(DSPARK_ERR_INVALID_ARG, "weight %d has no name", i);
    byname[table[i].name] = &table[i];
  }
  dspark_status err = DSPARK_OK;
  auto mat = [&](const std::string& name, int64_t rows, int64_t cols, Mat& m) {
    if (err) return;
    auto it = byname.find(name);
    if (it == byname.end()) { err = fail(DSPARK_ERR_SHAPE, "missing tensor %s", name.c_str()); return; }
    const dspark_weight& w = *it->second;
    if (w.rows != rows || w.cols != cols) {
      err = fail(DSPARK_ERR_SHAPE, "%s: shape [%lld, %lld], expected [%lld, %lld]", name.c_str(), (long long)w.rows,
                 (long long)w.cols, (long long)rows, (long long)cols);
      return;
    }
    if (w.dtype != c.weight_dtype) { err = fail(DSPARK_ERR_SHAPE, "%s: dtype %d, expected %d", name.c_str(), w.dtype, c.weight_dtype); return; }
    if (!w.data || (w.dtype == DSPARK_Q4 && (!w.scales || !w.biases))) {
      err = fail(DSPARK_ERR_INVALID_ARG, "%s: null device pointer", name.c_str());
      return;
    }
    m.kind = w.dtype == DSPARK_F32 ? WK_F32 : (w.dtype == DSPARK_BF16 ? WK_BF16 : WK_Q4);
    m.w = w.data;
    m.s = w.scales;
    m.b = w.biases;
    m.rows = rows;
    m.cols = cols;
  };
  auto vec = [&](const std::string& name, int64_t len) -> const void* {
    if (err) return nullptr;
    auto it = byname.find(name);
    if (it == byname.end()) { err = fail(DSPARK_ERR_SHAPE, "missing tensor %s", name.c_str()); return nullptr; }
    const dspark_weight& w = *it->second;
    if (w.rows * w.cols != len) { err = fail(DSPARK_ERR_SHAPE, "%s: %lld elements, expected %lld", name.c_str(), (long long)(w.rows * w.cols), (long long)len); return nullptr; }
    if (w.dtype != c.act_dtype) { err = fail(DSPARK_ERR_SHAPE, "%s: dtype %d, expected act dtype %d", name.c_str(), w.dtype, c.act_dtype); return nullptr; }
    if (!w.data) { err = fail(DSPARK_ERR_INVALID_ARG, "%s: null device pointer", name.c_str()); return nullptr; }
    return w.data;
  };
  dspark_model* m = new dspark_model();
  m->c = c;
  const int H = c.hidden_size, hd = c.global_head_dim, nH = c.num_attention_heads, nKv = c.num_global_key_value_heads;
  mat("embed_tokens.weight", c.vocab_size, H, m->embed);
  mat("lm_head.weight", c.vocab_size, H, m->lm);
  m->norm = vec("norm.weight", H);
  if (c.fc_in > 0) {
    mat("fc.weight", H, c.fc_in, m->fc);
    m->hidden_norm = vec("hidden_norm.weight", H);
  }
  if (c.markov_rank > 0) {
    mat("markov_head.markov_w1.weight", c.vocab_size, c.markov_rank, m->w1);
    mat("markov_head.markov_w2.weight", c.vocab_size, c.markov_rank, m->w2);
    if (c.markov_head_rnn) {
      mat("markov_head.rnn_wh.weight", c.markov_rank, c.markov_rank, m->wh);
      m->bh = vec("markov_head.rnn_bh.bias", c.markov_rank);
      m->rnn = true;
    }
  }
  if (c.enable_confidence_head) {
    mat("confidence_head.proj.weight", 1, H + (c.confidence_head_with_markov ? c.markov_rank : 0), m->conf);
    m->conf_b = vec("confidence_head.proj.bias", 1);
  }
  for (int i = 0; i < c.num_hidden_layers && !err; ++i) {
    const std::string p = "layers." + std::to_string(i) + ".";
    LayerW l{};
    mat(p + "self_attn.q_proj.weight", (int64_t)nH * hd, H, l.q);
    mat(p + "self_attn.k_proj.weight", (int64_t)nKv * hd, H, l.k);
    mat(p + "self_attn.o_proj.weight", H, (int64_t)nH * hd, l.o);
    mat(p + "mlp.gate_proj.weight", c.intermediate_size, H, l.g);
    mat(p + "mlp.up_proj.weight", c.intermediate_size, H, l.u);
    mat(p + "mlp.down_proj.weight", H, c.intermediate_size, l.d);
    l.qn = vec(p + "self_attn.q_norm.weight", hd);
    l.kn = vec(p + "self_attn.k_norm.weight", hd);
    l.in = vec(p + "input_layernorm.weight", H);
    l.pa = vec(p + "post_attention_layernorm.weight", H);
    l.pf = vec(p + "pre_feedforward_layernorm.weight", H);
    l.pff = vec(p + "post_feedforward_layernorm.weight", H);
    l.scalar = vec(p + "layer_scalar", 1);
    m->L.push_back(l);
  }
  if (err) {
    delete m;
    return err;
  }
  const int rotated = (int)std::floor(hd * c.partial_rotary_factor);
  m->nrot = (rotated + 1) / 2;  // pairs k with k < rotated / 2
  if (m->nrot > hd / 2) m->nrot = hd / 2;
  m->nq = (nH / nKv) * c.block_size;
  *out = m;
  return DSPARK_OK;
}

void dspark_model_destroy(dspark_model* m) { delete m; }

dspark_status dspark_model_set_tall_rows(dspark_model* m, int rows) {
  g_err.clear();
  if (!m) return fail(DSPARK_ERR_INVALID_ARG, "null model");
  m->tall_rows = rows > 0 ? rows : 0;
  return DSPARK_OK;
}

size_t dspark_model_aux_bytes(const dspark_model* m) {
  if (!m) return 0;
  return align256(((size_t)m->c.vocab_size + 1) * 4);
}

dspark_status dspark_model_prepare(dspark_model* m, void* aux_dev, size_t aux_bytes, hipStream_t stream) {
  g_err.clear();
  if (!m || !aux_dev) return fail(DSPARK_ERR_INVALID_ARG, "null model or aux buffer");
  if (aux_bytes < dspark_model_aux_bytes(m)) return fail(DSPARK_ERR_WORKSPACE, "aux buffer too small");
  if (m->c.markov_rank == 0) return DSPARK_OK;
  HIPCHECK(hipMemsetAsync((char*)aux_dev + (size_t)m->c.vocab_size * 4, 0, 4, stream));
  AuxArgs a;
  a.V = m->c.vocab_size;
  a.rank = m->c.markov_rank;
  a.wkind = m->w1.kind;
  a.group = m->c.group_size;
  a.w1 = m->w1.w; a.w1s = m->w1.s; a.w1b = m->w1.b;
  a.w2 = m->w2.w; a.w2s = m->w2.s; a.w2b = m->w2.b;
  a.aux = (float*)aux_dev;
  a.rnn = m->rnn ? 1 : 0;
  HIPCHECK(launch_aux(a, stream));
  return DSPARK_OK;
}

size_t dspark_project_workspace_bytes(const dspark_model* m, int input_kind, int B, int L) {
  if (!m || B <= 0 || L <= 0) return 0;
  return proj_layout(m, input_kind, B, L).total;
}

dspark_status dspark_project_context_kv(const dspark_model* m, int input_kind, const void* x_dev, int B, int L,
                                        const int32_t* pos0_host, void* const* k_out_dev, void* const* v_out_dev,
                                        void* ws_dev, size_t ws_bytes, hipStream_t stream) {
  g_err.clear();
  if (!m || !x_dev || !pos0_host || !v_out_dev || !ws_dev) return fail(DSPARK_ERR_INVALID_ARG, "null argument");
  if (B <= 0 || L <= 0) return fail(DSPARK_ERR_INVALID_ARG, "B and L must be positive");
  if (B > MAX_ROWS) return fail(DSPARK_ERR_UNSUPPORTED, "B > %d not built", MAX_ROWS);
  if ((int64_t)B * L > (1 << 24)) return fail(DSPARK_ERR_UNSUPPORTED, "B*L too large");
  if (input_kind != DSPARK_INPUT_CONTEXT_HIDDEN && input_kind != DSPARK_INPUT_TARGET_FEATURES)
    return fail(DSPARK_ERR_INVALID_ARG, "unknown input kind %d", input_kind);
  const dspark_config& c = m->c;
  if (input_kind == DSPARK_INPUT_TARGET_FEATURES && c.fc_in == 0)
    return fail(DSPARK_ERR_UNSUPPORTED, "model has no fc / hidden_norm");
  for (int b = 0; b < B; ++b)
    if (pos0_host[b] < 0) return fail(DSPARK_ERR_INVALID_ARG, "pos0[%d] < 0", b);
  for (int l = 0; l < c.num_hidden_layers; ++l)
    if ((k_out_dev && !k_out_dev[l]) || !v_out_dev[l])
      return fail(DSPARK_ERR_INVALID_ARG, "null K/V output for layer %d", l);
  const ProjLayout p = proj_layout(m, input_kind, B, L);
  if (ws_bytes < p.total) return fail(DSPARK_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, p.total);
  if ((uintptr_t)ws_dev & 255) return fail(DSPARK_ERR_WORKSPACE, "workspace must be 256-byte aligned");

  char* ws = (char*)ws_dev;
  const int M = B * L, H = c.hidden_size, hd = c.global_head_dim, nKv = c.num_global_key_value_heads;
  // reduction counters, zeroed here: the workspace may hold other data (a
  // call of another input kind or shape lays it out differently)
  unsigned* cnt = (unsigned*)(ws + p.cnt);
  const bool feats = input_kind == DSPARK_INPUT_TARGET_FEATURES;
  // counters are used by fc's split-K reduction and by a context projection
  // that splits K or runs its K/V epilogue in the last-arriving workgroup
  bool need_cnt = feats && p.fc.tall == TALL_NONE;
  for (int l0 = 0; l0 < c.num_hidden_layers; l0 += p.lay_per_gemm) {
    const int nl = std::min(p.lay_per_gemm, c.num_hidden_layers - l0);
    const GemmPlan gp = nl == p.lay_per_gemm ? p.kp : plan_gemm(c.weight_dtype, p.kp.xmode, M, nl * nKv * hd, H, hd,
                                                                 m->tall_rows);
    if (gp.tall == TALL_NONE && !kv_deferred(gp)) need_cnt = true;
  }
  if (need_cnt) HIPCHECK(timed("zero_counters", stream, [&] { return launch_zero(cnt, (int64_t)p.cwords, stream); }));
  TallBufs tb;
  tb.xop = (uint16_t*)(ws + p.xop);
  tb.T = (float*)(ws + p.T);
  NormIn nin{};
  bool fc_planes = false;  // k_proj's input planes written by fc's epilogue
  bool kp_all_planes = true;  // every k_proj launch reads hi / lo planes on the tiled path
  for (int l0 = 0; l0 < c.num_hidden_layers; l0 += p.lay_per_gemm) {
    const int nl = std::min(p.lay_per_gemm, c.num_hidden_layers - l0);
    const GemmPlan gp = nl == p.lay_per_gemm ? p.kp : plan_gemm(c.weight_dtype, p.kp.xmode, M, nl * nKv * hd, H, hd,
                                                                 m->tall_rows);
    if (gp.tall == TALL_NONE || gp.np != 2) kp_all_planes = false;
  }
  if (feats) {
    // fc rows and their statistics; k_proj reads hidden_norm(fc x)
    GemmArgs g{};
    g.X = x_dev;
    g.ldx = c.fc_in;
    g.M = M;
    g.N = H;
    g.K = c.fc_in;
    g.nseg = 1;
    g.seg[0] = seg_of(m->fc, 0);
    g.P = (float*)(ws + p.P);
    EpiArgs e{};
    e.Y = (float*)(ws + p.C);
    e.cnt = cnt;
    e.act_bf16 = act_bf16(m);
    e.h = nullptr;
    e.ldy = H;
    e.w1 = m->hidden_norm;
    e.sums = (RowStats*)(ws + p.sums);
    // both GEMMs tiled: fc's epilogue forms k_proj's input planes,
    // hidden_norm(fc x), itself (no statistics pass, no input preparation)
    SumsPrepArgs sp{};
    sp.w1 = m->hidden_norm;
    sp.act_bf16 = act_bf16(m);
    sp.eps = (float)c.rms_norm_eps;
    sp.xop = tb.xop;
    sp.plane = (int64_t)M * H;
    fc_planes = p.fc.tall != TALL_NONE && kp_all_planes && H <= SP_KMAX && H % 8 == 0;
    HIPCHECK(timed("gemm.fc", stream, [&] {
      return run_gemm(p.fc, g, e, EPI_SUMS, m->fc.kind, stream, tb, false, fc_planes ? &sp : nullptr);
    }));
    nin.y = e.Y;
    nin.sums = e.sums;
    nin.ld = H;
    nin.nparts = H / 64;
    nin.w1 = m->hidden_norm;
    nin.sc = nullptr;  // residual scale 1
    nin.eps = (float)c.rms_norm_eps;
    nin.act_bf16 = act_bf16(m);
  }
  for (int l0 = 0; l0 < c.num_hidden_layers; l0 += p.lay_per_gemm) {
    const int nl = std::min(p.lay_per_gemm, c.num_hidden_layers - l0);
    GemmArgs g{};
    g.X = x_dev;
    g.ldx = H;
    g.M = M;
    g.N = nl * nKv * hd;
    g.K = H;
    g.nseg = nl;
    for (int i = 0; i < nl; ++i) g.seg[i] = seg_of(m->L[l0 + i].k, i * nKv * hd);
    g.P = (float*)(ws + p.P);
    g.nin = nin;
    GemmPlan gp = p.kp;
    if (nl != p.lay_per_gemm) gp = plan_gemm(c.weight_dtype, p.kp.xmode, M, g.N, H, hd, m->tall_rows);
    EpiArgs e{};
    e.Y = (float*)(ws + p.Y);
    e.cnt = cnt;
    e.group_cols = hd;
    e.eps = (float)c.rms_norm_eps;
    e.act_bf16 = act_bf16(m);
    e.nH = c.num_attention_heads;
    e.nKv = nKv;
    e.hd = hd;
    e.L = L;
    e.rope = rope_of(m);
    for (int b = 0; b < B; ++b) e.pos0[b] = pos0_host[b];
    for (int i = 0; i < nl; ++i) {
      e.kn_l[i] = m->L[l0 + i].kn;
      e.kout[i] = k_out_dev ? k_out_dev[l0 + i] : nullptr;  // null: V-only cache
      e.vout[i] = v_out_dev[l0 + i];
    }
    HIPCHECK(timed("gemm.k_proj", stream, [&] {
      return run_gemm(gp, g, e, EPI_KV, m->L[l0].k.kind, stream, tb, fc_planes);
    }));
  }
  return DSPARK_OK;
}

size_t dspark_draft_workspace_bytes(const dspark_model* m, int A, int max_ctx, int64_t total_ctx) {
  if (!m || A <= 0 || A > MAX_ROWS || max_ctx < 0 || total_ctx < 0 || total_ctx > (int64_t)A * max_ctx) return 0;
  return draft_layout(m, A, true, total_ctx).total;
}

}  // extern "C"

namespace {

// dspark_draft_rows on the caller's workspace (use_scratch false), or on this
// device's fixed scratch array (use_scratch true; ws_dev and ws_bytes unused)
dspark_status draft_rows_impl(const dspark_model* m, int A, const void* const* k_ctx_dev,
                              const void* const* v_ctx_dev, const int32_t* ctx_len_host,
                              const int32_t* anchors_host, const int32_t* positions_host, int32_t* tokens_dev,
                              float* logits_dev, const void* aux_dev, void* ws_dev, size_t ws_bytes,
                              hipStream_t stream, bool use_scratch, const float* thresholds_host = nullptr,
                              float* conf_dev = nullptr, int32_t* lengths_dev = nullptr, bool allow_vonly = false,
                              const int32_t* ctx_pos0_host = nullptr, float temperature = 0.f,
                              const uint64_t* seeds_host = nullptr) {
  g_err.clear();
  const bool vonly = allow_vonly && !k_ctx_dev;  // a V-only context cache
  if (!m || (!k_ctx_dev && !vonly) || !v_ctx_dev || !ctx_len_host || !anchors_host || !positions_host ||
      !tokens_dev || (!ws_dev && !use_scratch))
    return fail(DSPARK_ERR_INVALID_ARG, "null argument");
  if (!(temperature >= 0.f) || temperature > 1e30f)  // NaN or infinite
    return fail(DSPARK_ERR_INVALID_ARG, "temperature must be finite and >= 0");
  const bool head = m->c.enable_confidence_head != 0;
  if (conf_dev && !head) return fail(DSPARK_ERR_INVALID_ARG, "confidence requested from a model without the head");
  const bool need_conf = head && (conf_dev || lengths_dev);
  const dspark_config& c = m->c;
  if (A <= 0) return fail(DSPARK_ERR_INVALID_ARG, "A must be positive");
  if (A > MAX_ROWS) return fail(DSPARK_ERR_UNSUPPORTED, "A > %d not built", MAX_ROWS);
  if (c.markov_rank > 0 && !aux_dev) return fail(DSPARK_ERR_INVALID_ARG, "aux buffer required when markov_rank > 0");
  const int G = c.block_size, nL = c.num_hidden_layers;
  RowTab rows{};
  rows.A = A;
  rows.gamma = G;
  int64_t total_keys = 0;
  for (int a = 0; a < A; ++a) {
    if (ctx_len_host[a] < 0) return fail(DSPARK_ERR_INVALID_ARG, "ctx_len[%d] < 0", a);
    if (ctx_len_host[a] > (1 << 24)) return fail(DSPARK_ERR_SHAPE, "ctx_len[%d] too large", a);
    if (anchors_host[a] < 0 || anchors_host[a] >= c.vocab_size)
      return fail(DSPARK_ERR_INVALID_ARG, "anchor %d of row %d out of range", anchors_host[a], a);
    if (positions_host[a] < 0) return fail(DSPARK_ERR_INVALID_ARG, "position[%d] < 0", a);
    rows.anchor[a] = anchors_host[a];
    rows.pos[a] = positions_host[a];
    rows.len[a] = ctx_len_host[a];
    total_keys += ctx_len_host[a] + G;
    for (int l = 0; l < nL; ++l)
      if (ctx_len_host[a] > 0 && ((!vonly && !k_ctx_dev[l * A + a]) || !v_ctx_dev[l * A + a]))
        return fail(DSPARK_ERR_INVALID_ARG, "null context K/V for layer %d row %d", l, a);
    if (ctx_pos0_host && ctx_pos0_host[a] < 0) return fail(DSPARK_ERR_INVALID_ARG, "ctx_pos0[%d] < 0", a);
  }
  if (vonly && c.act_dtype != DSPARK_BF16)
    return fail(DSPARK_ERR_UNSUPPORTED, "a V-only context cache is built for bf16 caches");
  // sampling keeps the noisy scores in the workspace's logits buffer
  const bool sampled = temperature > 0.f;
  const DraftLayout d = draft_layout(m, A, logits_dev == nullptr || sampled, total_keys - (int64_t)A * G);
  if (use_scratch) {
    if (d.total > NOALLOC_SCRATCH_BYTES)
      return fail(DSPARK_ERR_WORKSPACE,
                  "this round needs %zu bytes of scratch, above the %zu-byte fixed array of "
                  "dspark_draft_rows_noalloc (use dspark_draft_rows with a workspace)",
                  d.total, NOALLOC_SCRATCH_BYTES);
    const dspark_status sst = scratch_address(&ws_dev);
    if (sst) return sst;
    ws_bytes = NOALLOC_SCRATCH_BYTES;
  }
  if (ws_bytes < d.total) return fail(DSPARK_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, d.total);
  if ((uintptr_t)ws_dev & 255) return fail(DSPARK_ERR_WORKSPACE, "workspace must be 256-byte aligned");

  char* ws = (char*)ws_dev;
  const int M = A * G, H = c.hidden_size, I = c.intermediate_size, hd = c.global_head_dim;
  const int nH = c.num_attention_heads, nKv = c.num_global_key_value_heads;
  const float eps = (float)c.rms_norm_eps;
  const int abf = act_bf16(m);
  float* hA = (float*)(ws + d.hA);  // the embedding, then each layer's post-attention residual
  float* hB = (float*)(ws + d.hB);  // the residual entering each layer
  float* Y = (float*)(ws + d.Y);
  RowStats* sums = (RowStats*)(ws + d.sums);
  float2* rt = (float2*)(ws + d.rt);
  float* O = (float*)(ws + d.O);
  float* act = (float*)(ws + d.act);
  float* P = (float*)(ws + d.P);
  unsigned* cnt = (unsigned*)(ws + d.cnt);
  const int wk = m->lm.kind;
  const int NC = nc_of(m);
  TallBufs tb;
  tb.xop = (uint16_t*)(ws + d.xop);
  tb.T = (float*)(ws + d.T);

  // attention split plan: context splits of `split` keys, then the block split
  const int64_t total_ctx = total_keys - (int64_t)A * G;
  const bool wide = total_ctx >= ATTN_WIDE_MIN_KEYS && attn_wide_ok(m->nq, hd);
  if (vonly && !attn_vonly_ok(m->nq, hd, wide))
    return fail(DSPARK_ERR_UNSUPPORTED, "a V-only context cache is not built for head_dim %d with %d query rows",
                hd, m->nq);
  const int split = wide ? attn_split_wide(total_ctx, A) : attn_split(total_ctx);
  AttnArgs at{};
  at.vonly = vonly ? 1 : 0;
  at.rope_step = std::pow((double)c.rope_theta, -2.0 / c.global_head_dim);
  at.nrot = m->nrot;
  for (int a = 0; a < A; ++a) at.ctx_pos0[a] = ctx_pos0_host ? ctx_pos0_host[a] : 0;
  MergeArgs mg{};
  int nsplit = 0;
  for (int a = 0; a < A; ++a) {
    at.split_off[a] = nsplit;
    nsplit += ceil_div(ctx_len_host[a], split) + 1;
    at.len[a] = ctx_len_host[a];
  }
  at.split_off[A] = nsplit;
  if (nsplit > d.nsplit_max) return fail(DSPARK_ERR_SHAPE, "attention splits %d exceed the plan", nsplit);
  // wide kernel: the splits of row a on XCD a mod 8 when that keeps the
  // eight XCDs' shares within a quarter of the even share
  int attn_grid = nsplit;
  if (wide && A >= 8) {
    int load[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int a = 0; a < A; ++a) load[a & 7] += at.split_off[a + 1] - at.split_off[a];
    const int mx = *std::max_element(load, load + 8);
    if (4 * 8 * (int64_t)mx <= 5 * (int64_t)nsplit) {
      at.xcd_rows = 1;
      attn_grid = 8 * mx;
    }
  }
  std::memcpy(mg.split_off, at.split_off, sizeof at.split_off);
  at.A = A;
  at.gamma = G;
  at.nKv = nKv;
  at.nH = nH;
  at.nq = m->nq;
  at.split = split;
  at.M = M;
  at.hd = hd;
  at.eps = eps;
  at.q = (const float*)(ws + d.q);
  at.kb = (const float*)(ws + d.kb);
  at.vb = (const float*)(ws + d.vb);
  at.ssq = (const float*)(ws + d.ssq);
  at.opart = ws + d.opart;
  at.ml = (float*)(ws + d.ml);
  mg.A = A;
  mg.gamma = G;
  mg.nKv = nKv;
  mg.nq = m->nq;
  mg.nH = nH;
  mg.hd = hd;
  mg.opart = at.opart;
  mg.part_f16 = c.act_dtype == DSPARK_BF16 ? 1 : 0;  // the attention kernels' KVB variant
  mg.lane_order = wide ? 1 : 0;                         // the wide kernel stores fp16 partials in lane order
  mg.ml = at.ml;
  mg.O = O;
  mg.ldo = d.ldo;
  // a tiled o projection over hi + lo planes reads them straight from the merge
  const bool o_planes = d.o.tall != TALL_NONE && d.o.np == 2;
  if (o_planes) {
    mg.planes = tb.xop;
    mg.plane = (int64_t)M * nH * hd;
  }

  EmbedArgs em{};
  em.E = m->embed.w;
  em.Es = m->embed.s;
  em.Eb = m->embed.b;
  em.ekind = m->embed.kind;
  em.group = c.group_size;
  em.H = H;
  em.scale = (float)std::sqrt((double)H);
  em.mask_id = c.mask_token_id;
  em.h = hA;
  em.ldh = d.ldh;
  em.act_bf16 = abf;
  em.nL = nL;
  for (int l = 0; l < nL; ++l) em.scal_src[l] = m->L[l].scalar;
  float* scal = (float*)(ws + d.scal);  // scal[0] = 1, scal[1 + l] = layer l's scalar
  em.scal = scal;
  em.sums = sums;
  em.rt = rt;
  em.rope = rope_of(m);
  em.cnt = cnt;
  em.ncnt = (int)d.cwords;
  em.rows = rows;
  HIPCHECK(timed("embed", stream, [&] { return launch_embed(em, M, stream); }));

  // input rows of a GEMM: x = rms((h + rms(y) w1) sc) w2 from the statistics
  auto norm_in = [&](const float* h, const float* y, const void* w1, const float* sc, const void* w2, float* hout) {
    NormIn n{};
    n.h = h;
    n.y = y;
    n.sums = sums;
    n.nparts = H / 64;
    n.w1 = w1;
    n.w2 = w2;
    n.sc = sc;
    n.hout = hout;
    n.ld = d.ldh;
    n.eps = eps;
    n.act_bf16 = abf;
    return n;
  };

  EpiArgs e{};
  e.cnt = cnt;
  e.eps = eps;
  e.act_bf16 = abf;
  e.nH = nH;
  e.nKv = nKv;
  e.hd = hd;
  e.gamma = G;
  e.rt = rt;
  e.q = (float*)(ws + d.q);
  e.kb = (float*)(ws + d.kb);
  e.vb = (float*)(ws + d.vb);
  e.ssq = (float*)(ws + d.ssq);
  e.act = act;
  e.ld_act = d.ldact;
  e.ldy = d.ldh;
  e.sums = sums;

  // The residual stream is formed lazily: a sublayer output y stays in Y
  // with its row statistics, and the next GEMM's staging adds it to the
  // residual it read and writes the sum (q|k writes hB, gate|up writes hA).
  // the tiled o and down projections form the next GEMM's input planes in
  // their epilogue when that GEMM is tiled too (no separate preparation)
  auto sums_next = [&](const float* h, const void* w1, const float* sc, const void* w2, float* hout) {
    SumsPrepArgs sp{};
    sp.h = h;
    sp.ldh = d.ldh;
    sp.w1 = w1;
    sp.sc = sc;
    sp.w2 = w2;
    sp.act_bf16 = abf;
    sp.eps = eps;
    sp.hout = hout;
    sp.xop = tb.xop;
    sp.plane = (int64_t)M * H;
    return sp;
  };
  const bool fuse_prep = H <= SP_KMAX && H % 8 == 0;
  bool planes_ready = false;  // the next GEMM's input planes are already in tb.xop
  const float* y_prev = nullptr;  // pending sublayer output folded into the next input norm
  const void* w1_prev = nullptr;
  const float* sc_prev = scal;
  for (int l = 0; l < nL; ++l) {
    const LayerW& W = m->L[l];
    GemmArgs g{};
    g.ldx = H;
    g.M = M;
    g.N = (nH + nKv) * hd;
    g.K = H;
    g.nseg = 2;
    g.seg[0] = seg_of(W.q, 0);
    g.seg[1] = seg_of(W.k, nH * hd);
    g.P = P;
    g.nin = norm_in(hA, y_prev, w1_prev, sc_prev, W.in, hB);
    e.qn = W.qn;
    e.kn = W.kn;
    HIPCHECK(timed("gemm.qk", stream, [&] { return run_gemm(d.qk, g, e, EPI_QK, wk, stream, tb, planes_ready); }));
    planes_ready = false;

    for (int a = 0; a < A; ++a) {
      at.row[a].k = vonly ? nullptr : k_ctx_dev[l * A + a];
      at.row[a].v = v_ctx_dev[l * A + a];
    }
    at.kn = W.kn;  // a V-only cache rebuilds the context keys with this layer's k_norm
    HIPCHECK(timed("attn", stream, [&] {
      return wide ? launch_attn_wide(at, c.act_dtype == DSPARK_BF16, attn_grid, stream)
                  : launch_attn(at, c.act_dtype == DSPARK_BF16, nsplit, stream);
    }));
    HIPCHECK(timed("attn_merge", stream, [&] { return launch_merge(mg, stream); }));

    g = GemmArgs{};
    g.X = O;
    g.ldx = d.ldo;
    g.M = M;
    g.N = H;
    g.K = nH * hd;
    g.nseg = 1;
    g.seg[0] = seg_of(W.o, 0);
    g.P = P;
    e.Y = Y;
    e.h = hB;
    e.w1 = W.pa;
    const bool fuse_o = fuse_prep && d.o.tall != TALL_NONE && d.gu.tall != TALL_NONE;
    const SumsPrepArgs nx_o = sums_next(hB, W.pa, scal, W.pf, hA);
    HIPCHECK(timed("gemm.o", stream, [&] {
      return run_gemm(d.o, g, e, EPI_SUMS, wk, stream, tb, o_planes, fuse_o ? &nx_o : nullptr);
    }));

    g = GemmArgs{};
    g.ldx = H;
    g.M = M;
    g.N = 2 * I;
    g.K = H;
    g.nseg = 2;
    g.seg[0] = seg_of(W.g, 0);
    g.seg[1] = seg_of(W.u, I);
    g.P = P;
    g.nin = norm_in(hB, Y, W.pa, scal, W.pf, hA);
    if (d.dn_planes) {
      e.act_planes = (uint16_t*)(ws + d.xop2);
      e.act_plane = (int64_t)M * I;
    }
    HIPCHECK(timed("gemm.gate_up", stream, [&] { return run_gemm(d.gu, g, e, EPI_GELU, wk, stream, tb, fuse_o); }));

    g = GemmArgs{};
    g.X = act;
    g.ldx = d.ldact;
    g.M = M;
    g.N = H;
    g.K = I;
    g.nseg = 1;
    g.seg[0] = seg_of(W.d, 0);
    g.P = P;
    e.Y = Y;
    e.h = hA;
    e.w1 = W.pff;
    TallBufs tb_dn = tb;
    if (d.dn_planes) tb_dn.xop = (uint16_t*)(ws + d.xop2);
    // the next GEMM: the next layer's q|k, or lm_head (whose hn rows feed
    // the confidence head)
    const bool last = l + 1 == nL;
    const bool fuse_d = fuse_prep && d.dn.tall != TALL_NONE && (last ? d.lm.tall : d.qk.tall) != TALL_NONE &&
                        (!d.dn_planes || tb_dn.xop != tb.xop);
    const SumsPrepArgs nx_d = sums_next(hA, W.pff, scal + 1 + l, last ? m->norm : m->L[l + 1].in,
                                        last ? (need_conf ? hB : nullptr) : hB);
    HIPCHECK(timed("gemm.down", stream, [&] {
      return run_gemm(d.dn, g, e, EPI_SUMS, wk, stream, tb_dn, d.dn_planes, fuse_d ? &nx_d : nullptr);
    }));
    planes_ready = fuse_d;
    y_prev = Y;
    w1_prev = W.pff;
    sc_prev = scal + 1 + l;
  }

  GemmArgs g{};
  g.ldx = H;
  g.M = M;
  g.N = c.vocab_size;
  g.K = H;
  g.nseg = 1;
  g.seg[0] = seg_of(m->lm, 0);
  g.P = P;
  // the confidence head reads the final residual rows (hB is free by now)
  g.nin = norm_in(hA, y_prev, w1_prev, sc_prev, m->norm, need_conf ? hB : nullptr);
  float* z = logits_dev ? logits_dev : (float*)(ws + d.z);
  e.Y = z;
  e.cap = c.final_logit_softcapping > 0 ? (float)c.final_logit_softcapping : 0.f;
  e.aux = c.markov_rank > 0 ? (const float*)aux_dev : nullptr;
  e.lohi = (float2*)(ws + d.lohi);
  e.NC = NC;
  if (sampled) {
    e.smp.temperature = temperature;
    e.smp.gamma = G;
    e.smp.zs = (float*)(ws + d.z);
    for (int a = 0; a < A; ++a) e.smp.seeds[a] = seeds_host ? seeds_host[a] : 0ull;
  }
  HIPCHECK(timed("gemm.lm_head", stream, [&] { return run_gemm(d.lm, g, e, EPI_LM, wk, stream, tb, planes_ready); }));

  WalkArgs w{};
  w.rows = rows;
  w.V = c.vocab_size;
  w.NC = NC;
  w.rank = c.markov_rank;
  w.wkind = m->w1.kind;
  w.group = c.group_size;
  w.z = sampled ? e.smp.zs : z;  // the walk draws from the noisy scores when sampling
  w.lohi = e.lohi;
  w.aux = e.aux;
  w.w1 = m->w1.w; w.w1s = m->w1.s; w.w1b = m->w1.b;
  w.w2 = m->w2.w; w.w2s = m->w2.s; w.w2b = m->w2.b;
  w.rnn = m->rnn ? 1 : 0;
  w.wh = m->wh.w; w.whs = m->wh.s; w.whb = m->wh.b;
  w.bh = m->bh;
  w.act_bf16 = abf;
  w.tokens = tokens_dev;
  HIPCHECK(timed("markov_walk", stream, [&] { return launch_walk(w, stream); }));

  if (conf_dev || lengths_dev) {
    ConfArgs cf{};
    cf.rows = rows;
    cf.head = need_conf ? 1 : 0;
    cf.H = H;
    cf.rank = c.markov_rank;
    cf.with_markov = c.confidence_head_with_markov ? 1 : 0;
    cf.wkind = m->conf.kind;
    cf.group = c.group_size;
    cf.act_bf16 = abf;
    cf.hn = hB;
    cf.ldh = d.ldh;
    cf.wnorm = m->norm;
    cf.eps = eps;
    cf.pw = m->conf.w; cf.ps = m->conf.s; cf.pb = m->conf.b;
    cf.bias = m->conf_b;
    cf.w1 = m->w1.w; cf.w1s = m->w1.s; cf.w1b = m->w1.b;
    cf.tokens = tokens_dev;
    for (int k = 0; k < G; ++k)
      cf.thr[k] = thresholds_host ? thresholds_host[k] : (float)c.confidence_threshold;
    cf.conf = conf_dev ? conf_dev : (float*)(ws + d.conf);
    cf.lengths = lengths_dev;
    HIPCHECK(timed("confidence", stream, [&] { return launch_conf(cf, stream); }));
  }
  return DSPARK_OK;
}

}  // namespace

extern "C" {

dspark_status dspark_draft_rows(const dspark_model* m, int A, const void* const* k_ctx_dev,
                                const void* const* v_ctx_dev, const int32_t* ctx_len_host,
                                const int32_t* anchors_host, const int32_t* positions_host, int32_t* tokens_dev,
                                float* logits_dev, const void* aux_dev, void* ws_dev, size_t ws_bytes,
                                hipStream_t stream) {
  return draft_rows_impl(m, A, k_ctx_dev, v_ctx_dev, ctx_len_host, anchors_host, positions_host, tokens_dev,
                         logits_dev, aux_dev, ws_dev, ws_bytes, stream, false);
}

dspark_status dspark_draft_rows_conf(const dspark_model* m, int A, const void* const* k_ctx_dev,
                                     const void* const* v_ctx_dev, const int32_t* ctx_len_host,
                                     const int32_t* anchors_host, const int32_t* positions_host,
                                     const float* thresholds_host, int32_t* tokens_dev, float* logits_dev,
                                     float* conf_dev, int32_t* lengths_dev, const void* aux_dev, void* ws_dev,
                                     size_t ws_bytes, hipStream_t stream) {
  return draft_rows_impl(m, A, k_ctx_dev, v_ctx_dev, ctx_len_host, anchors_host, positions_host, tokens_dev,
                         logits_dev, aux_dev, ws_dev, ws_bytes, stream, false, thresholds_host, conf_dev,
                         lengths_dev);
}

dspark_status dspark_draft_rows_ex(const dspark_model* m, const dspark_draft_args* x, void* ws_dev, size_t ws_bytes,
                                   hipStream_t stream) {
  g_err.clear();
  if (!x) return fail(DSPARK_ERR_INVALID_ARG, "null arguments");
  return draft_rows_impl(m, x->A, x->k_ctx_dev, x->v_ctx_dev, x->ctx_len_host, x->anchors_host, x->positions_host,
                         x->tokens_dev, x->logits_dev, x->aux_dev, ws_dev, ws_bytes, stream, false,
                         x->thresholds_host, x->conf_dev, x->lengths_dev, true, x->ctx_pos0_host, x->temperature,
                         x->seeds_host);
}

dspark_status dspark_draft_rows_noalloc(const dspark_model* m, int A, const void* const* k_ctx_dev,
                                        const void* const* v_ctx_dev, const int32_t* ctx_len_host,
                                        const int32_t* anchors_host, const int32_t* positions_host,
                                        int32_t* tokens_dev, float* logits_dev, const void* aux_dev,
                                        hipStream_t stream) {
  return draft_rows_impl(m, A, k_ctx_dev, v_ctx_dev, ctx_len_host, anchors_host, positions_host, tokens_dev,
                         logits_dev, aux_dev, nullptr, 0, stream, true);
}

size_t dspark_draft_noalloc_max_bytes(void) { return NOALLOC_SCRATCH_BYTES; }

dspark_status dspark_draft_block(const dspark_model* m, const void* const* k_ctx_dev, const void* const* v_ctx_dev,
                                 int32_t ctx_len, int32_t anchor, int32_t position, int32_t* tokens_dev,
                                 float* logits_dev, const void* aux_dev, void* ws_dev, size_t ws_bytes,
                                 hipStream_t stream) {
  return dspark_draft_rows(m, 1, k_ctx_dev, v_ctx_dev, &ctx_len, &anchor, &position, tokens_dev, logits_dev, aux_dev,
                           ws_dev, ws_bytes, stream);
}

}  // extern "C"
