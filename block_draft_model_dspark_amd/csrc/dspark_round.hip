// Row-wise kernels of the draft round: scaled embedding, the GEMM epilogues
// (RMSNorm, RoPE, residual, GELU-gate, softcap), and the context K/V epilogue.
//
// Each epilogue first sums the split-K partials P[s][m][n] of its GEMM.  All
// arithmetic is fp32; RoPE angles are formed in double (positions reach
// 32k+, where an fp32 angle would be off by ~1e-3 rad).
#include "dspark_kernels.hpp"
#include "dspark_common.hpp"

namespace dsp {

__device__ __forceinline__ float sum_parts(const float* P, int S, int M, int N, int m, int n) {
  float v = 0.f;
  for (int s = 0; s < S; ++s) v += P[((int64_t)s * M + m) * N + n];
  return v;
}

// embedding row of a table in f32 / bf16 / q4 storage, element k
__device__ __forceinline__ float table_elem(const void* E, const void* Es, const void* Eb, int kind, int group,
                                            int64_t row, int cols, int k) {
  if (kind == WK_F32) return ((const float*)E)[row * cols + k];
  if (kind == WK_BF16) return bf2f(((const uint16_t*)E)[row * cols + k]);
  const uint32_t w = ((const uint32_t*)E)[row * (cols >> 3) + (k >> 3)];
  const float q = (float)((w >> (4 * (k & 7))) & 0xFu);
  const int64_t gi = row * (cols / group) + k / group;
  return bf2f(((const uint16_t*)Es)[gi]) * q + bf2f(((const uint16_t*)Eb)[gi]);
}

// ---------------------------------------------------------------------------
// deepspec.ts, #forwardBackbone: h = embed([anchor, MASK...]) * sqrt(H);
// x = input_layernorm(h) of layer 0.  grid M, block 256.
// ---------------------------------------------------------------------------
constexpr int EPT = 32;  // elements per thread of a 256-thread row kernel (H <= 8192)

__global__ __launch_bounds__(256) void k_embed(const EmbedArgs a) {
  __shared__ float red[8];
  const int m = blockIdx.x;
  const int row = m / a.rows.gamma, g = m - row * a.rows.gamma;
  const int64_t id = g == 0 ? a.rows.anchor[row] : a.mask_id;
  float v[EPT];
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int k = threadIdx.x + 256 * e;
    v[e] = 0.f;
    if (k < a.H) {
      v[e] = table_elem(a.E, a.Es, a.Eb, a.ekind, a.group, id, a.H, k) * a.scale;
      a.h[(int64_t)m * a.H + k] = v[e];
      ss += v[e] * v[e];
    }
  }
  const float r = 1.f / sqrtf(block_sum(ss, red) / a.H + a.eps);
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int k = threadIdx.x + 256 * e;
    if (k < a.H) a.x[(int64_t)m * a.H + k] = v[e] * r * ld_act(a.w_in, k, a.act_bf16);
  }
}

// ---------------------------------------------------------------------------
// deepspec.ts, #forwardBackbone q / block-k path:
//   q = RoPE(q_norm(q_proj x), p+g); v_b = rms(k_proj x); k_b = RoPE(k_norm(k_proj x), p+g)
// grid (M, nH + nKv), block hd
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_qk_epi(const QkEpiArgs a) {
  __shared__ float red[8];
  __shared__ float buf[256];
  const int m = blockIdx.x, head = blockIdx.y, d = threadIdx.x, hd = a.hd, half = hd >> 1;
  const int row = m / a.rows.gamma, g = m - row * a.rows.gamma;
  const int col = head * hd + d;  // q heads first, then the kv heads
  const float y = sum_parts(a.P, a.S, a.M, a.N, m, col);
  const float r = 1.f / sqrtf(block_sum(y * y, red) / hd + a.eps);
  const int64_t pos = (int64_t)a.rows.pos[row] + g;
  float c, s;
  rope_cs(pos, d < half ? d : d - half, hd, a.rope.theta, a.rope.nrot, c, s);
  const int rep = a.nH / a.nKv;
  const int nq = rep * a.rows.gamma;
  if (head < a.nH) {
    const float yn = y * r * ld_act(a.qn, d, a.act_bf16);
    buf[d] = yn;
    __syncthreads();
    const float o = d < half ? yn * c - buf[d + half] * s : yn * c + buf[d - half] * s;
    const int kvh = head / rep, hl = head - kvh * rep;
    a.q[(((int64_t)row * a.nKv + kvh) * nq + hl * a.rows.gamma + g) * hd + d] = o;
  } else {
    const int kvh = head - a.nH;
    const float vn = y * r;
    const int64_t off = (((int64_t)row * a.nKv + kvh) * a.rows.gamma + g) * hd + d;
    a.vb[off] = vn;
    const float kn = vn * ld_act(a.kn, d, a.act_bf16);
    buf[d] = kn;
    __syncthreads();
    a.kb[off] = d < half ? kn * c - buf[d + half] * s : kn * c + buf[d - half] * s;
  }
}

// ---------------------------------------------------------------------------
// split-softmax merge: O = sum_s e^{m_s - M} O_s / sum_s e^{m_s - M} l_s
// grid A*nKv*nq, block hd
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_merge(const MergeArgs a) {
  const int idx = blockIdx.x;
  const int j = idx % a.nq, kvh = (idx / a.nq) % a.nKv, row = idx / (a.nq * a.nKv);
  const int s0 = a.split_off[row], s1 = a.split_off[row + 1];
  float mx = -INFINITY;
  for (int s = s0; s < s1; ++s) mx = fmaxf(mx, a.ml[(((int64_t)s * a.nKv + kvh) * a.nq + j) * 2]);
  float den = 0.f, num = 0.f;
  for (int s = s0; s < s1; ++s) {
    const int64_t b = ((int64_t)s * a.nKv + kvh) * a.nq + j;
    const float w = expf(a.ml[b * 2] - mx);
    den += w * a.ml[b * 2 + 1];
    num += w * a.opart[b * a.hd + threadIdx.x];
  }
  const int rep = a.nH / a.nKv, hl = j / a.gamma, g = j - hl * a.gamma;
  const int h = kvh * rep + hl;
  a.O[((int64_t)row * a.gamma + g) * (a.nH * a.hd) + h * a.hd + threadIdx.x] = num / den;
}

// ---------------------------------------------------------------------------
// row epilogues (grid M, block 256):
//  mode 0, deepspec.ts #forwardBackbone after attention:
//     h += post_attention_layernorm(o); x = pre_feedforward_layernorm(h)
//  mode 1, after the MLP:
//     h = (h + post_feedforward_layernorm(d)) * layer_scalar; x = next norm(h)
//  mode 2, deepspec.ts #projectContext: x = hidden_norm(fc out)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_row_epi(const RowEpiArgs a) {
  __shared__ float red[8];
  const int m = blockIdx.x, N = a.N;
  float y[EPT];
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int k = threadIdx.x + 256 * e;
    y[e] = k < N ? sum_parts(a.P, a.S, a.M, N, m, k) : 0.f;
    ss += y[e] * y[e];
  }
  float r = 1.f / sqrtf(block_sum(ss, red) / N + a.eps);
  if (a.mode == 2) {
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int k = threadIdx.x + 256 * e;
      if (k < N) a.x[(int64_t)m * N + k] = y[e] * r * ld_act(a.w1, k, a.act_bf16);
    }
    return;
  }
  const float scal = a.mode == 1 ? ld_act(a.scalar, 0, a.act_bf16) : 1.f;
  float ss2 = 0.f;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int k = threadIdx.x + 256 * e;
    if (k < N) {
      const int64_t o = (int64_t)m * N + k;
      const float hn = (a.h[o] + y[e] * r * ld_act(a.w1, k, a.act_bf16)) * scal;
      a.h[o] = hn;
      y[e] = hn;
      ss2 += hn * hn;
    }
  }
  r = 1.f / sqrtf(block_sum(ss2, red) / N + a.eps);
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int k = threadIdx.x + 256 * e;
    if (k < N) a.x[(int64_t)m * N + k] = y[e] * r * ld_act(a.w2, k, a.act_bf16);
  }
}

// deepspec.ts, #geluTanhMlp: act = gelu_tanh(gate x) * up x.  P columns are
// [gate | up], N = 2I.  grid ceil(M*I/256), block 256
__global__ __launch_bounds__(256) void k_gateup(const GateUpArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)a.M * a.I) return;
  const int m = (int)(idx / a.I), i = (int)(idx - (int64_t)m * a.I);
  const float gt = sum_parts(a.P, a.S, a.M, 2 * a.I, m, i);
  const float up = sum_parts(a.P, a.S, a.M, 2 * a.I, m, a.I + i);
  a.x[idx] = gelu_tanh(gt) * up;
}

// ---------------------------------------------------------------------------
// deepspec.ts, #computeLogits: z = cap * tanh(lm_head(h) / cap), plus the
// per-chunk statistics the walk prunes with.  For a step, any prev token
// gives |markov_w2[v] . markov_w1[prev]| <= ||w2_v|| * max ||w1|| =: B_v, so
// a vocabulary entry with z_v + B_v below max_u (z_u - B_u) can never win.
// Per (row, 256-entry chunk): lo = max (z - B) and the WALK_TOP best z + B.
// grid (NC, M), block 256
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_lm_epi(const LmEpiArgs a) {
  __shared__ float redu[4];
  __shared__ int redi[4];
  const int c = blockIdx.x, m = blockIdx.y;
  const int v = c * WALK_CHUNK + threadIdx.x;
  float z = -INFINITY, bnd = 0.f;
  if (v < a.V) {
    z = sum_parts(a.P, a.S, a.M, a.V, m, v);
    if (a.cap > 0.f) z = a.cap * tanhf(z / a.cap);
    a.z[(int64_t)m * a.V + v] = z;
    if (a.aux) bnd = a.aux[v] * a.aux[a.V] * (1.f + 1e-5f);
  }
  const float lov = z - bnd;
  const float lom = block_max(lov, redu);
  float hv = z + bnd;
  float2* top = a.top + ((int64_t)m * a.NC + c) * WALK_TOP;
  for (int t = 0; t < WALK_TOP; ++t) {
    float u = hv;
    int i = v < a.V ? v : 0x7fffffff;
    block_argmax(u, i, redu, redi);
    if (threadIdx.x == 0) top[t] = make_float2(u, __int_as_float(i));
    if (v == i) hv = -INFINITY;
    __syncthreads();
  }
  if (threadIdx.x == 0) a.lo[(int64_t)m * a.NC + c] = lom;
}

// markov_w1 / markov_w2 element (table_elem with the head's own storage)
__device__ __forceinline__ float head_elem(const void* w, const void* s, const void* b, int kind, int group,
                                           int64_t row, int cols, int k) {
  return table_elem(w, s, b, kind, group, row, cols, k);
}

// ---------------------------------------------------------------------------
// deepspec.ts, draftRows sequential walk at temperature 0:
//   prev = anchor; for k < gamma: tok = argmax(z[k] + markov_w2 markov_w1[prev]); prev = tok
// One workgroup per draft row.  Only entries that survive the bound test
// (k_lm_epi) are scored; a chunk whose WALK_TOP-th best still passes is
// scored in full.  Ties go to the lower index.
// grid A, block 256
// ---------------------------------------------------------------------------
constexpr int WALK_CAP = 3 * 1024;  // NC <= 1024 chunks, < WALK_TOP candidates each otherwise

__global__ __launch_bounds__(256) void k_walk(const WalkArgs a) {
  __shared__ float redu[4];
  __shared__ int redi[4];
  __shared__ int cand[WALK_CAP];
  __shared__ int ovf[1024];
  __shared__ float e[256];
  __shared__ int ncand, novf, prev_s;
  const int row = blockIdx.x, tid = threadIdx.x, G = a.rows.gamma;
  if (tid == 0) prev_s = a.rows.anchor[row];
  for (int k = 0; k < G; ++k) {
    const int64_t m = (int64_t)row * G + k;
    float lm = -INFINITY;
    for (int c = tid; c < a.NC; c += 256) lm = fmaxf(lm, a.lo[m * a.NC + c]);
    lm = block_max(lm, redu);
    const float thr = lm - 1e-4f * (1.f + fabsf(lm));
    if (tid == 0) { ncand = 0; novf = 0; }
    __syncthreads();
    const int prev = prev_s;
    for (int c = tid; c < a.NC; c += 256) {
      const float2* tp = a.top + (m * a.NC + c) * WALK_TOP;
      if (tp[WALK_TOP - 1].x >= thr) {
        ovf[atomicAdd(&novf, 1)] = c;
      } else {
        for (int t = 0; t < WALK_TOP - 1; ++t)
          if (tp[t].x >= thr) cand[atomicAdd(&ncand, 1)] = __float_as_int(tp[t].y);
      }
    }
    if (a.rank > 0)
      for (int j = tid; j < a.rank; j += 256)
        e[j] = head_elem(a.w1, a.w1s, a.w1b, a.wkind, a.group, prev, a.rank, j);
    __syncthreads();
    float bu = -INFINITY;
    int bi = 0x7fffffff;
    const int nc = ncand, no = novf;
    const int tot = nc + no * WALK_CHUNK;
    for (int i = tid; i < tot; i += 256) {
      int v;
      if (i < nc) v = cand[i];
      else {
        const int q = i - nc;
        v = ovf[q / WALK_CHUNK] * WALK_CHUNK + (q % WALK_CHUNK);
        if (v >= a.V) continue;
      }
      float u = a.z[m * a.V + v];
      if (a.rank > 0) {
        float dot = 0.f;
        for (int j = 0; j < a.rank; ++j) dot += head_elem(a.w2, a.w2s, a.w2b, a.wkind, a.group, v, a.rank, j) * e[j];
        u += dot;
      }
      if (better(u, v, bu, bi)) { bu = u; bi = v; }
    }
    block_argmax(bu, bi, redu, redi);
    if (tid == 0) {
      // no finite candidate (non-finite logits): report -1 and keep a valid row index
      const bool ok = bi >= 0 && bi < a.V;
      a.tokens[m] = ok ? bi : -1;
      prev_s = ok ? bi : 0;
    }
    __syncthreads();
  }
}

// per-model walk bound data: aux[v] = ||markov_w2[v]||, aux[V] = max ||markov_w1[v]||
// (aux[V] zeroed by the caller).  grid ceil(V/4), block 256 (one wave per row)
__global__ __launch_bounds__(256) void k_aux(const AuxArgs a) {
  const int v = blockIdx.x * 4 + (threadIdx.x >> 6), l = threadIdx.x & 63;
  if (v >= a.V) return;
  float s2 = 0.f, s1 = 0.f;
  for (int j = l; j < a.rank; j += 64) {
    const float x2 = head_elem(a.w2, a.w2s, a.w2b, a.wkind, a.group, v, a.rank, j);
    const float x1 = head_elem(a.w1, a.w1s, a.w1b, a.wkind, a.group, v, a.rank, j);
    s2 += x2 * x2;
    s1 += x1 * x1;
  }
  s2 = wave_sum(s2);
  s1 = wave_sum(s1);
  if (l == 0) {
    a.aux[v] = sqrtf(s2) * (1.f + 1e-5f);
    atomicMax((unsigned int*)&a.aux[a.V], __float_as_uint(sqrtf(s1) * (1.f + 1e-5f)));
  }
}

// ---------------------------------------------------------------------------
// deepspec.ts, #projectContextKVRows epilogue: per (context row, layer, kv head)
//   V = rms(k) (no weight, no RoPE); K = RoPE(rms(k) * k_norm, pos0 + i)
// grid (M = B*L, layers*nKv), block hd
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_kv_epi(const KvEpiArgs a) {
  __shared__ float red[8];
  __shared__ float buf[256];
  const int m = blockIdx.x, lh = blockIdx.y, d = threadIdx.x, hd = a.hd, half = hd >> 1;
  const int layer = lh / a.nKv, kvh = lh - layer * a.nKv;
  const int b = m / a.L, i = m - b * a.L;
  const float y = sum_parts(a.P, a.S, a.M, a.N, m, lh * hd + d);
  const float vn = y / sqrtf(block_sum(y * y, red) / hd + a.eps);
  const int64_t off = (((int64_t)b * a.nKv + kvh) * a.L + i) * hd + d;
  st_act(a.vout[layer], off, vn, a.act_bf16);
  const float kn = vn * ld_act(a.kn[layer], d, a.act_bf16);
  buf[d] = kn;
  __syncthreads();
  float c, s;
  rope_cs((int64_t)a.pos0[b] + i, d < half ? d : d - half, hd, a.rope.theta, a.rope.nrot, c, s);
  st_act(a.kout[layer], off, d < half ? kn * c - buf[d + half] * s : kn * c + buf[d - half] * s, a.act_bf16);
}

// ---------------------------------------------------------------------------
hipError_t launch_embed(const EmbedArgs& a, int M, hipStream_t st) {
  hipLaunchKernelGGL(k_embed, dim3(M), dim3(256), 0, st, a);
  return hipGetLastError();
}
hipError_t launch_qk_epi(const QkEpiArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_qk_epi, dim3(a.M, a.nH + a.nKv), dim3(a.hd), 0, st, a);
  return hipGetLastError();
}
hipError_t launch_merge(const MergeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_merge, dim3(a.A * a.nKv * a.nq), dim3(a.hd), 0, st, a);
  return hipGetLastError();
}
hipError_t launch_row_epi(const RowEpiArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_row_epi, dim3(a.M), dim3(256), 0, st, a);
  return hipGetLastError();
}
hipError_t launch_gateup(const GateUpArgs& a, hipStream_t st) {
  const int64_t n = (int64_t)a.M * a.I;
  hipLaunchKernelGGL(k_gateup, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}
hipError_t launch_lm_epi(const LmEpiArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_lm_epi, dim3(a.NC, a.M), dim3(256), 0, st, a);
  return hipGetLastError();
}
hipError_t launch_walk(const WalkArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_walk, dim3(a.rows.A), dim3(256), 0, st, a);
  return hipGetLastError();
}
hipError_t launch_aux(const AuxArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_aux, dim3((a.V + 3) / 4), dim3(256), 0, st, a);
  return hipGetLastError();
}
hipError_t launch_kv_epi(const KvEpiArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_kv_epi, dim3(a.M, a.layers * a.nKv), dim3(a.hd), 0, st, a);
  return hipGetLastError();
}

}  // namespace dsp
