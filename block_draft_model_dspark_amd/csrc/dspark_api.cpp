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
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// run `launch` (returning hipError_t), bracketed by events when timing is on
template <class F>
hipError_t timed(const char* name, hipStream_t st, F&& launch) {
  if (!g_prof) return launch();
  ProfEntry e{name, prof_event(), prof_event()};
  if (e.a) hipEventRecord(e.a, st);
  hipError_t r = launch();
  if (e.b) hipEventRecord(e.b, st);
  if (e.a && e.b) g_prof_log.push_back(e);
  return r;
}
int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

}  // namespace

struct dspark_model {
  dspark_config c;
  Mat embed, fc, lm, w1, w2;
  const void* hidden_norm = nullptr;
  const void* norm = nullptr;
  std::vector<LayerW> L;
  int nrot = 0;
  int nq = 0;
};

namespace {

int act_bf16(const dspark_model* m) { return m->c.act_dtype == DSPARK_BF16 ? 1 : 0; }
int nc_of(const dspark_model* m) { return ceil_div(m->c.vocab_size, WALK_CHUNK); }

RopeCfg rope_of(const dspark_model* m) {
  RopeCfg r;
  r.theta = m->c.rope_theta;
  r.hd = m->c.global_head_dim;
  r.nrot = m->nrot;
  return r;
}

// ---- GEMM planning --------------------------------------------------------
struct GemmPlan {
  int mt, kc, S, kslice;
  size_t pbytes;
};

GemmPlan plan_gemm(int wk, bool xbf, int M, int N, int K) {
  GemmPlan p;
  // row tiles per workgroup: 1 for M <= 16, else 4 (2 and 3 are not enabled)
  p.mt = M <= 16 ? 1 : 4;
  int kc = wk == WK_F32 ? 256 : 512;
  while (kc > 128 && gemm_lds_bytes(wk, xbf, p.mt, kc) > 65536) kc /= 2;
  const int mblocks = ceil_div(M, 16 * p.mt);
  const int ntw = ceil_div(N / 16, 4);
  if (M <= 64) {
    // split K so the weight stream spreads over >= 512 workgroups
    while (kc > 128 && (int64_t)ntw * mblocks * ceil_div(K, kc) < 512) kc /= 2;
    if (kc > K) kc = K;
    p.kc = kc;
    p.kslice = kc;
    p.S = ceil_div(K, kc);
  } else {
    if (kc > K) kc = K;
    p.kc = kc;
    p.S = 1;
    p.kslice = ceil_div(K, kc) * kc;
  }
  p.pbytes = (size_t)p.S * M * N * 4;
  return p;
}

hipError_t run_gemm(const GemmPlan& p, GemmArgs a, int wk, bool xbf, hipStream_t st) {
  a.kslice = p.kslice;
  a.kc = p.kc;
  return launch_gemm(a, wk, xbf, p.mt, p.S, st);
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
struct DraftLayout {
  size_t h, x, P, q, kb, vb, opart, ml, z, lo, top, total;
  GemmPlan qk, o, gu, dn, lm;
};

int attn_split(int64_t total_keys) {
  int64_t s = (total_keys + 511) / 512;
  s = (s + 31) / 32 * 32;
  return (int)std::max<int64_t>(64, s);
}

DraftLayout draft_layout(const dspark_model* m, int A, bool with_z) {
  const dspark_config& c = m->c;
  const int M = A * c.block_size, H = c.hidden_size, I = c.intermediate_size, hd = c.global_head_dim;
  const int wk = c.weight_dtype;
  DraftLayout d;
  d.qk = plan_gemm(wk, false, M, (c.num_attention_heads + c.num_global_key_value_heads) * hd, H);
  d.o = plan_gemm(wk, false, M, H, c.num_attention_heads * hd);
  d.gu = plan_gemm(wk, false, M, 2 * I, H);
  d.dn = plan_gemm(wk, false, M, H, I);
  d.lm = plan_gemm(wk, false, M, c.vocab_size, H);
  const size_t pmax = std::max({d.qk.pbytes, d.o.pbytes, d.gu.pbytes, d.dn.pbytes, d.lm.pbytes});
  const int xw = std::max({H, I, c.num_attention_heads * hd});
  const int nsplit_max = 512 + A;
  const int NC = nc_of(m);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  d.h = take((size_t)M * H * 4);
  d.x = take((size_t)M * xw * 4);
  d.P = take(pmax);
  d.q = take((size_t)A * c.num_global_key_value_heads * m->nq * hd * 4);
  d.kb = take((size_t)A * c.num_global_key_value_heads * c.block_size * hd * 4);
  d.vb = take((size_t)A * c.num_global_key_value_heads * c.block_size * hd * 4);
  d.opart = take((size_t)nsplit_max * c.num_global_key_value_heads * m->nq * hd * 4);
  d.ml = take((size_t)nsplit_max * c.num_global_key_value_heads * m->nq * 2 * 4);
  d.z = with_z ? take((size_t)M * c.vocab_size * 4) : 0;
  d.lo = take((size_t)M * NC * 4);
  d.top = take((size_t)M * NC * WALK_TOP * 8);
  d.total = off;
  return d;
}

// ---- projection workspace layout -----------------------------------------
struct ProjLayout {
  size_t P1, C, P2, total;
  GemmPlan fc, kp;
  int lay_per_gemm;
};

ProjLayout proj_layout(const dspark_model* m, int input_kind, int B, int L) {
  const dspark_config& c = m->c;
  const int M = B * L, H = c.hidden_size;
  ProjLayout p{};
  p.lay_per_gemm = std::min(c.num_hidden_layers, MAX_SEG);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  const bool in_bf16 = c.act_dtype == DSPARK_BF16;
  if (input_kind == DSPARK_INPUT_TARGET_FEATURES) {
    p.fc = plan_gemm(c.weight_dtype, in_bf16, M, H, c.fc_in);
    p.P1 = take(p.fc.pbytes);
    p.C = take((size_t)M * H * 4);
    p.kp = plan_gemm(c.weight_dtype, false, M, p.lay_per_gemm * c.num_global_key_value_heads * c.global_head_dim, H);
  } else {
    p.kp = plan_gemm(c.weight_dtype, in_bf16, M, p.lay_per_gemm * c.num_global_key_value_heads * c.global_head_dim, H);
  }
  p.P2 = take(p.kp.pbytes);
  p.total = off;
  return p;
}

// ---- model creation --------------------------------------------------------
dspark_status check_config(const dspark_config& c) {
  if (!c.attention_k_eq_v)
    return fail(DSPARK_ERR_UNSUPPORTED, "attention_k_eq_v=false needs a v_proj path; only V == K is implemented");
  if (c.markov_rank > 0 && !c.markov_head_vanilla)
    return fail(DSPARK_ERR_UNSUPPORTED, "only the vanilla Markov head is implemented");
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
  if (c.vocab_size % 16 || c.vocab_size > 1024 * WALK_CHUNK)
    return fail(DSPARK_ERR_UNSUPPORTED, "vocab_size must be a multiple of 16 and at most %d", 1024 * WALK_CHUNK);
  if (c.block_size > 32) return fail(DSPARK_ERR_UNSUPPORTED, "block_size > 32 not built");
  if ((c.num_attention_heads / c.num_global_key_value_heads) * c.block_size > 128)
    return fail(DSPARK_ERR_UNSUPPORTED, "more than 128 query rows per kv head not built");
  if (c.markov_rank > 256 || c.markov_rank % 8)
    return fail(DSPARK_ERR_UNSUPPORTED, "markov_rank must be a multiple of 8 and at most 256");
  if (c.mask_token_id < 0 || c.mask_token_id >= c.vocab_size)
    return fail(DSPARK_ERR_INVALID_ARG, "mask_token_id out of range");
  if (!(c.rope_theta > 0) || !(c.partial_rotary_factor >= 0 && c.partial_rotary_factor <= 1) || !(c.rms_norm_eps >= 0))
    return fail(DSPARK_ERR_INVALID_ARG, "rope_theta, partial_rotary_factor or rms_norm_eps out of range");
  if (c.act_dtype != DSPARK_F32 && c.act_dtype != DSPARK_BF16)
    return fail(DSPARK_ERR_UNSUPPORTED, "act_dtype must be F32 or BF16");
  if (c.weight_dtype != DSPARK_F32 && c.weight_dtype != DSPARK_BF16 && c.weight_dtype != DSPARK_Q4)
    return fail(DSPARK_ERR_UNSUPPORTED, "weight_dtype must be F32, BF16 or Q4");
  if (c.weight_dtype == DSPARK_Q4) {
    // The first GPU run of a 4-bit round faulted and no cause has been shown
    // yet; the path stays switched off until one is.
    return fail(DSPARK_ERR_UNSUPPORTED, "4-bit weights are disabled in this build (GPU fault under analysis)");
    if (c.group_size != 64) return fail(DSPARK_ERR_UNSUPPORTED, "Q4 group size %d not built (64)", c.group_size);
    if (c.markov_rank % 64) return fail(DSPARK_ERR_UNSUPPORTED, "Q4 Markov tables need rank %% 64 == 0");
  }
  return DSPARK_OK;
}

}  // namespace

extern "C" {

const char* dspark_last_error(void) { return g_err.c_str(); }

void dspark_profile_enable(int on) { g_prof = on != 0; }

int dspark_profile_read(dspark_kernel_time* out, int max) {
  std::vector<dspark_kernel_time> acc;
  for (const ProfEntry& e : g_prof_log) {
    float ms = 0.f;
    hipEventSynchronize(e.b);
    hipEventElapsedTime(&ms, e.a, e.b);
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
  if (!m || !x_dev || !pos0_host || !k_out_dev || !v_out_dev || !ws_dev)
    return fail(DSPARK_ERR_INVALID_ARG, "null argument");
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
    if (!k_out_dev[l] || !v_out_dev[l]) return fail(DSPARK_ERR_INVALID_ARG, "null K/V output for layer %d", l);
  const ProjLayout p = proj_layout(m, input_kind, B, L);
  if (ws_bytes < p.total) return fail(DSPARK_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, p.total);
  if ((uintptr_t)ws_dev & 255) return fail(DSPARK_ERR_WORKSPACE, "workspace must be 256-byte aligned");

  char* ws = (char*)ws_dev;
  const int M = B * L, H = c.hidden_size, hd = c.global_head_dim, nKv = c.num_global_key_value_heads;
  const bool in_bf16 = c.act_dtype == DSPARK_BF16;
  const void* X = x_dev;
  bool xbf = in_bf16;
  if (input_kind == DSPARK_INPUT_TARGET_FEATURES) {
    GemmArgs g{};
    g.X = x_dev;
    g.ldx = c.fc_in;
    g.M = M;
    g.N = H;
    g.K = c.fc_in;
    g.nseg = 1;
    g.seg[0] = seg_of(m->fc, 0);
    g.P = (float*)(ws + p.P1);
    HIPCHECK(timed("gemm.fc", stream, [&] { return run_gemm(p.fc, g, m->fc.kind, in_bf16, stream); }));
    RowEpiArgs r{};
    r.P = g.P;
    r.S = p.fc.S;
    r.M = M;
    r.N = H;
    r.w1 = m->hidden_norm;
    r.act_bf16 = act_bf16(m);
    r.eps = (float)c.rms_norm_eps;
    r.x = (float*)(ws + p.C);
    r.mode = 2;
    HIPCHECK(timed("norm.hidden", stream, [&] { return launch_row_epi(r, stream); }));
    X = r.x;
    xbf = false;
  }
  for (int l0 = 0; l0 < c.num_hidden_layers; l0 += p.lay_per_gemm) {
    const int nl = std::min(p.lay_per_gemm, c.num_hidden_layers - l0);
    GemmArgs g{};
    g.X = X;
    g.ldx = H;
    g.M = M;
    g.N = nl * nKv * hd;
    g.K = H;
    g.nseg = nl;
    for (int i = 0; i < nl; ++i) g.seg[i] = seg_of(m->L[l0 + i].k, i * nKv * hd);
    g.P = (float*)(ws + p.P2);
    GemmPlan gp = p.kp;
    if (nl != p.lay_per_gemm) gp = plan_gemm(c.weight_dtype, xbf, M, g.N, H);
    HIPCHECK(timed("gemm.k_proj", stream, [&] { return run_gemm(gp, g, m->L[l0].k.kind, xbf, stream); }));
    KvEpiArgs e{};
    e.P = g.P;
    e.S = gp.S;
    e.M = M;
    e.N = g.N;
    e.B = B;
    e.L = L;
    e.layers = nl;
    e.nKv = nKv;
    e.hd = hd;
    e.eps = (float)c.rms_norm_eps;
    e.act_bf16 = act_bf16(m);
    e.rope = rope_of(m);
    for (int b = 0; b < B; ++b) e.pos0[b] = pos0_host[b];
    for (int i = 0; i < nl; ++i) {
      e.kn[i] = m->L[l0 + i].kn;
      e.kout[i] = k_out_dev[l0 + i];
      e.vout[i] = v_out_dev[l0 + i];
    }
    HIPCHECK(timed("kv_epilogue", stream, [&] { return launch_kv_epi(e, stream); }));
  }
  return DSPARK_OK;
}

size_t dspark_draft_workspace_bytes(const dspark_model* m, int A, int max_ctx, int64_t total_ctx) {
  (void)max_ctx;
  (void)total_ctx;
  if (!m || A <= 0 || A > MAX_ROWS) return 0;
  return draft_layout(m, A, true).total;
}

dspark_status dspark_draft_rows(const dspark_model* m, int A, const void* const* k_ctx_dev,
                                const void* const* v_ctx_dev, const int32_t* ctx_len_host,
                                const int32_t* anchors_host, const int32_t* positions_host, int32_t* tokens_dev,
                                float* logits_dev, const void* aux_dev, void* ws_dev, size_t ws_bytes,
                                hipStream_t stream) {
  g_err.clear();
  if (!m || !k_ctx_dev || !v_ctx_dev || !ctx_len_host || !anchors_host || !positions_host || !tokens_dev || !ws_dev)
    return fail(DSPARK_ERR_INVALID_ARG, "null argument");
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
      if (ctx_len_host[a] > 0 && (!k_ctx_dev[l * A + a] || !v_ctx_dev[l * A + a]))
        return fail(DSPARK_ERR_INVALID_ARG, "null context K/V for layer %d row %d", l, a);
  }
  const DraftLayout d = draft_layout(m, A, logits_dev == nullptr);
  if (ws_bytes < d.total) return fail(DSPARK_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, d.total);
  if ((uintptr_t)ws_dev & 255) return fail(DSPARK_ERR_WORKSPACE, "workspace must be 256-byte aligned");

  char* ws = (char*)ws_dev;
  const int M = A * G, H = c.hidden_size, I = c.intermediate_size, hd = c.global_head_dim;
  const int nH = c.num_attention_heads, nKv = c.num_global_key_value_heads;
  const float eps = (float)c.rms_norm_eps;
  float* h = (float*)(ws + d.h);
  float* x = (float*)(ws + d.x);
  float* P = (float*)(ws + d.P);
  const int wk = m->lm.kind;

  // attention split plan
  const int split = attn_split(total_keys);
  AttnArgs at{};
  MergeArgs mg{};
  int nsplit = 0;
  for (int a = 0; a < A; ++a) {
    at.split_off[a] = nsplit;
    nsplit += ceil_div(ctx_len_host[a] + G, split);
    at.len[a] = ctx_len_host[a];
  }
  at.split_off[A] = nsplit;
  std::memcpy(mg.split_off, at.split_off, sizeof at.split_off);
  at.A = A;
  at.gamma = G;
  at.nKv = nKv;
  at.nq = m->nq;
  at.split = split;
  at.q = (const float*)(ws + d.q);
  at.kb = (const float*)(ws + d.kb);
  at.vb = (const float*)(ws + d.vb);
  at.opart = (float*)(ws + d.opart);
  at.ml = (float*)(ws + d.ml);
  mg.A = A;
  mg.gamma = G;
  mg.nKv = nKv;
  mg.nq = m->nq;
  mg.nH = nH;
  mg.hd = hd;
  mg.opart = at.opart;
  mg.ml = at.ml;
  mg.O = x;

  EmbedArgs e{};
  e.E = m->embed.w;
  e.Es = m->embed.s;
  e.Eb = m->embed.b;
  e.ekind = m->embed.kind;
  e.group = c.group_size;
  e.w_in = m->L[0].in;
  e.act_bf16 = act_bf16(m);
  e.H = H;
  e.eps = eps;
  e.scale = (float)std::sqrt((double)H);
  e.mask_id = c.mask_token_id;
  e.h = h;
  e.x = x;
  e.rows = rows;
  HIPCHECK(timed("embed", stream, [&] { return launch_embed(e, M, stream); }));

  for (int l = 0; l < nL; ++l) {
    const LayerW& W = m->L[l];
    GemmArgs g{};
    g.X = x;
    g.ldx = H;
    g.M = M;
    g.N = (nH + nKv) * hd;
    g.K = H;
    g.nseg = 2;
    g.seg[0] = seg_of(W.q, 0);
    g.seg[1] = seg_of(W.k, nH * hd);
    g.P = P;
    HIPCHECK(timed("gemm.qk", stream, [&] { return run_gemm(d.qk, g, wk, false, stream); }));

    QkEpiArgs q{};
    q.P = P;
    q.S = d.qk.S;
    q.M = M;
    q.N = g.N;
    q.qn = W.qn;
    q.kn = W.kn;
    q.act_bf16 = act_bf16(m);
    q.nH = nH;
    q.nKv = nKv;
    q.hd = hd;
    q.eps = eps;
    q.rope = rope_of(m);
    q.q = (float*)(ws + d.q);
    q.kb = (float*)(ws + d.kb);
    q.vb = (float*)(ws + d.vb);
    q.rows = rows;
    HIPCHECK(timed("qk_epilogue", stream, [&] { return launch_qk_epi(q, stream); }));

    for (int a = 0; a < A; ++a) {
      at.row[a].k = k_ctx_dev[l * A + a];
      at.row[a].v = v_ctx_dev[l * A + a];
    }
    HIPCHECK(timed("attn", stream, [&] { return launch_attn(at, hd, c.act_dtype == DSPARK_BF16, nsplit, stream); }));
    HIPCHECK(timed("attn_merge", stream, [&] { return launch_merge(mg, stream); }));

    g = GemmArgs{};
    g.X = x;
    g.ldx = nH * hd;
    g.M = M;
    g.N = H;
    g.K = nH * hd;
    g.nseg = 1;
    g.seg[0] = seg_of(W.o, 0);
    g.P = P;
    HIPCHECK(timed("gemm.o", stream, [&] { return run_gemm(d.o, g, wk, false, stream); }));
    RowEpiArgs r{};
    r.P = P;
    r.S = d.o.S;
    r.M = M;
    r.N = H;
    r.w1 = W.pa;
    r.w2 = W.pf;
    r.act_bf16 = act_bf16(m);
    r.eps = eps;
    r.h = h;
    r.x = x;
    r.mode = 0;
    HIPCHECK(timed("attn_out_epilogue", stream, [&] { return launch_row_epi(r, stream); }));

    g = GemmArgs{};
    g.X = x;
    g.ldx = H;
    g.M = M;
    g.N = 2 * I;
    g.K = H;
    g.nseg = 2;
    g.seg[0] = seg_of(W.g, 0);
    g.seg[1] = seg_of(W.u, I);
    g.P = P;
    HIPCHECK(timed("gemm.gate_up", stream, [&] { return run_gemm(d.gu, g, wk, false, stream); }));
    GateUpArgs gu{};
    gu.P = P;
    gu.S = d.gu.S;
    gu.M = M;
    gu.I = I;
    gu.x = x;
    HIPCHECK(timed("gelu_gate", stream, [&] { return launch_gateup(gu, stream); }));

    g = GemmArgs{};
    g.X = x;
    g.ldx = I;
    g.M = M;
    g.N = H;
    g.K = I;
    g.nseg = 1;
    g.seg[0] = seg_of(W.d, 0);
    g.P = P;
    HIPCHECK(timed("gemm.down", stream, [&] { return run_gemm(d.dn, g, wk, false, stream); }));
    r = RowEpiArgs{};
    r.P = P;
    r.S = d.dn.S;
    r.M = M;
    r.N = H;
    r.w1 = W.pff;
    r.w2 = l + 1 < nL ? m->L[l + 1].in : m->norm;
    r.scalar = W.scalar;
    r.act_bf16 = act_bf16(m);
    r.eps = eps;
    r.h = h;
    r.x = x;
    r.mode = 1;
    HIPCHECK(timed("mlp_out_epilogue", stream, [&] { return launch_row_epi(r, stream); }));
  }

  GemmArgs g{};
  g.X = x;
  g.ldx = H;
  g.M = M;
  g.N = c.vocab_size;
  g.K = H;
  g.nseg = 1;
  g.seg[0] = seg_of(m->lm, 0);
  g.P = P;
  HIPCHECK(timed("gemm.lm_head", stream, [&] { return run_gemm(d.lm, g, wk, false, stream); }));

  const int NC = nc_of(m);
  LmEpiArgs le{};
  le.P = P;
  le.S = d.lm.S;
  le.M = M;
  le.V = c.vocab_size;
  le.cap = c.final_logit_softcapping > 0 ? (float)c.final_logit_softcapping : 0.f;
  le.aux = c.markov_rank > 0 ? (const float*)aux_dev : nullptr;
  le.z = logits_dev ? logits_dev : (float*)(ws + d.z);
  le.lo = (float*)(ws + d.lo);
  le.top = (float2*)(ws + d.top);
  le.NC = NC;
  HIPCHECK(timed("logits_epilogue", stream, [&] { return launch_lm_epi(le, stream); }));

  WalkArgs w{};
  w.rows = rows;
  w.V = c.vocab_size;
  w.NC = NC;
  w.rank = c.markov_rank;
  w.wkind = m->w1.kind;
  w.group = c.group_size;
  w.z = le.z;
  w.lo = le.lo;
  w.top = le.top;
  w.w1 = m->w1.w; w.w1s = m->w1.s; w.w1b = m->w1.b;
  w.w2 = m->w2.w; w.w2s = m->w2.s; w.w2b = m->w2.b;
  w.tokens = tokens_dev;
  HIPCHECK(timed("markov_walk", stream, [&] { return launch_walk(w, stream); }));
  return DSPARK_OK;
}

dspark_status dspark_draft_block(const dspark_model* m, const void* const* k_ctx_dev, const void* const* v_ctx_dev,
                                 int32_t ctx_len, int32_t anchor, int32_t position, int32_t* tokens_dev,
                                 float* logits_dev, const void* aux_dev, void* ws_dev, size_t ws_bytes,
                                 hipStream_t stream) {
  return dspark_draft_rows(m, 1, k_ctx_dev, v_ctx_dev, &ctx_len, &anchor, &position, tokens_dev, logits_dev, aux_dev,
                           ws_dev, ws_bytes, stream);
}

}  // extern "C"
