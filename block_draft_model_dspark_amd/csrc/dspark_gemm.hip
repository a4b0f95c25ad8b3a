// Weight-streaming GEMM y = x . W^T on bf16 MFMA (v_mfma_f32_16x16x32_bf16)
// with the split-K reduction and the consumer's epilogue fused in.
//
// Used for every linear layer of the drafter (deepspec.ts, matmulW: x @ W^T
// with W kept in its [out, in] storage): q|k, o, gate|up, down, lm_head, fc
// and the per-layer k_proj of the context projection.
//
// Work split: a 256-thread workgroup = 4 wave64s; wave w owns one 16-column
// output tile of the workgroup's 64-column block (blockIdx.x), the workgroup
// owns one K slice (blockIdx.y) and one block of MT*16 rows (blockIdx.z);
// with 16-row tiles and several row blocks, (x, y, z) is renumbered so that
// the row blocks of a (column block, K slice) share its weight tile
// (stream_block_of).
// Each wave issues all weight loads of a K sub-slice straight from HBM into
// registers (16 B per lane per 32-wide k step: the B operand layout needs no
// shuffling), then the workgroup stages the activation sub-slice into LDS
// split into bf16 hi + lo halves in A-operand order, and the MFMAs run hi
// and lo against the same weight registers.  Activations are fp32 in HBM;
// hi + lo carries ~16 mantissa bits, which the draft round needs (scale-1
// attention amplifies input rounding).  bf16 inputs are exact in hi alone.
//
// Input rows (XM_NORM): the sandwich norms of the backbone are applied while
// staging, from the producer's per-64-column row statistics (NormIn), so no
// kernel ever walks a whole row alone:
//   hn = (h + rms(y) * w1) * sc,   x = rms(hn) * w2,
// with sum hn^2 = sc^2 (sum h^2 + 2 r1 sum h w1 y + r1^2 sum (w1 y)^2).
// Column block 0 also writes hn, the next residual.
//
// Weight kinds:
//   bf16: used as is.
//   f32 : split hi + lo as well; x_hi*w_hi + x_lo*w_hi + x_hi*w_lo.
//   q4  : affine 4-bit, groups of 64 along K.  Codes become the exact bf16
//         values 1 + q/16 with two bit operations per pair, and
//         sum_k x (s q + b) = 16 s * sum x (1 + q/16) + (b - 16 s) * sum x
//         is applied per group after the group's MFMAs.
//
// Reduction (no extra launch, deterministic): with S > 1 K slices every
// workgroup writes its partial tile, and the last one to arrive at its
// column block (counter) sums the S partials in slice order and runs the
// epilogue on its 64 columns.  Only the context K/V epilogue (a head's
// RMSNorm, which must be final in the cache) needs a second arrival per
// head.  Counters are zero on entry and are left zero.
#include <type_traits>

#include "dspark_kernels.hpp"
#include "dspark_common.hpp"

namespace dsp {

// eight 4-bit codes of one word -> bf16 values 1 + q/16; element order is
// codes 0,4,1,5,2,6,3,7 (the staging pass applies the same order to x)
__device__ __forceinline__ bf16x8 q4_decode(uint32_t w) {
  u32x4 r;
  r[0] = ((w << 3) & 0x00780078u) | 0x3F803F80u;
  r[1] = ((w >> 1) & 0x00780078u) | 0x3F803F80u;
  r[2] = ((w >> 5) & 0x00780078u) | 0x3F803F80u;
  r[3] = ((w >> 9) & 0x00780078u) | 0x3F803F80u;
  return __builtin_bit_cast(bf16x8, r);
}

// Split-K partials (and the reduced tile a head epilogue reads) may be
// written and read on different XCDs, whose L2 caches are not coherent with
// each other.  They are stored and loaded with agent-scope atomic accesses
// (per-access coherence bits, write-through / re-fetch at the device
// coherence point) instead of cache-wide L2 write-back and invalidate.
__device__ __forceinline__ void st_coh(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coh(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// true in the workgroup that is the `total`-th to arrive at *ctr (which it
// resets).  Every wave first drains its outstanding stores, so the
// workgroup's coherent stores are complete before the counter moves.
__device__ __forceinline__ bool arrive_last(unsigned* ctr, unsigned total, int* flag) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = old == total - 1;
    if (last) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = last;
  }
  __syncthreads();
  return *flag != 0;
}

// ---------------------------------------------------------------------------
// input rows (XM_NORM): per-row factors (r1, r2) and sc from the statistics
// ---------------------------------------------------------------------------
// The first 16 rows' statistics are loaded by norm_issue before the weight
// loads are issued, so that they do not wait behind the weights (a wave's
// loads complete in order).  Every thread issues the same fixed number of
// loads (indices clamped, surplus parts masked when summing): a load under a
// run-time condition would make the compiler wait for every load in flight.
// norm_finish reduces them; further 16-row tiles (MT > 1) load theirs there.
constexpr int NV = 2;  // parts each thread loads early (16 threads per row: K up to 16 * NV * 64 = 2048);
                       // norm_finish reads the parts of wider rows

__device__ __forceinline__ void norm_issue(const GemmArgs& g, int mbase, RowStats* v, float& sc, int vt) {
  const NormIn& n = g.nin;
  const int tid = vt, sub = tid & 15;
  const int m = min(mbase + (tid >> 4), g.M - 1);
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = n.sums[(int64_t)min(sub + 16 * i, n.nparts - 1) * g.M + m];
  sc = n.sc ? *n.sc : 1.f;
}

template <int MT>
__device__ __forceinline__ void norm_finish(const GemmArgs& g, int mbase, const RowStats* v0, float sc, float2* rs,
                                            int vt) {
  const NormIn& n = g.nin;
  const int tid = vt, sub = tid & 15;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int ml = 16 * t + (tid >> 4);
    const int m = min(mbase + ml, g.M - 1);
    RowStats s = {0.0, 0.0, 0.0, 0.0};
    int p0 = sub;
    if (t == 0) {
#pragma unroll
      for (int i = 0; i < NV; ++i)
        if (sub + 16 * i < n.nparts) {
          s.x += v0[i].x;
          s.y += v0[i].y;
          s.z += v0[i].z;
          s.w += v0[i].w;
        }
      p0 = sub + 16 * NV;
    }
    // (rows wider than the early loads cover, and further 16-row tiles; the
    // loads here wait for every load in flight, weights included)
    for (int p = p0; p < n.nparts; p += 16) {
      const RowStats v = n.sums[(int64_t)p * g.M + m];
      s.x += v.x;
      s.y += v.y;
      s.z += v.z;
      s.w += v.w;
    }
    s.x = row16_sum_d(s.x);
    s.y = row16_sum_d(s.y);
    s.z = row16_sum_d(s.z);
    s.w = row16_sum_d(s.w);
    if (sub == 0) {
      // rows past M: r2 = 0, so the staged input of such a row is zero
      const float2 f = norm_factors(s, sc, g.K, n.eps);
      rs[ml] = mbase + ml < g.M ? f : make_float2(f.x, 0.f);
    }
  }
  if (tid == 0) rs[MT * 16] = make_float2(sc, 0.f);
}

// ---------------------------------------------------------------------------
// epilogues on the workgroup's reduced tile (acc: wave's 16 columns, rows
// 16t + 4g + i of the row block)
// ---------------------------------------------------------------------------

// deepspec.ts, #forwardBackbone, q / block-k path of one head part:
//   q = RoPE(q_norm(q_proj x)), v_b = rms(k_proj x), k_b = RoPE(k_norm(k_proj x))
// The RMS factor of a head needs all hd columns; it is a per-row scalar that
// commutes with RoPE, so this stores RoPE(w * y) and y unscaled plus the
// part's sum y^2, and the attention kernel applies the factor.
template <int MT>
__device__ __forceinline__ void epi_qk(const GemmArgs& g, const EpiArgs& e, const f32x4* acc, int mbase, int cb, float* tile) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, gq = lane >> 4;
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) tile[(wave * MT * 16 + t * 16 + 4 * gq + i) * 16 + (lane & 15)] = acc[t][i];
  __syncthreads();
  const int hd = e.hd, half = hd >> 1, hj = hd >> 6, head = cb / hj, cp = cb - head * hj;
  const bool isq = head < e.nH;
  const void* nw = isq ? e.qn : e.kn;
  const int rep = e.nH / e.nKv, nq = rep * e.gamma;
  constexpr int IT = MT * 16 * 32 / 256;
  float ya[IT], yb[IT], wa[IT], wb[IT];
  float2 cs[IT];
#pragma unroll
  for (int u = 0; u < IT; ++u) {
    const int idx = tid + 256 * u, r = idx >> 5, j = idx & 31, d = 32 * cp + j;
    const int m = min(mbase + r, g.M - 1);
    wa[u] = ld_act_v(nw, d, e.act_bf16);
    wb[u] = ld_act_v(nw, d + half, e.act_bf16);
    cs[u] = e.rt[(int64_t)m * half + d];
    ya[u] = tile[((j >> 4) * MT * 16 + r) * 16 + (j & 15)];
    yb[u] = tile[((2 + (j >> 4)) * MT * 16 + r) * 16 + (j & 15)];
  }
#pragma unroll
  for (int u = 0; u < IT; ++u) {
    const int idx = tid + 256 * u, r = idx >> 5, j = idx & 31, d = 32 * cp + j;
    const int m = mbase + r;
    const float ta = ya[u] * wa[u], tb = yb[u] * wb[u];
    const float oa = ta * cs[u].x - tb * cs[u].y, ob = tb * cs[u].x + ta * cs[u].y;
    const float ss = half_sum(ya[u] * ya[u] + yb[u] * yb[u]);
    if (m < g.M) {
      const int arow = m / e.gamma, gs = m - arow * e.gamma;
      if (isq) {
        const int kvh = head / rep, hl = head - kvh * rep;
        float* dst = e.q + (((int64_t)arow * e.nKv + kvh) * nq + hl * e.gamma + gs) * hd;
        dst[d] = oa;
        dst[d + half] = ob;
      } else {
        const int kvh = head - e.nH;
        const int64_t off = (((int64_t)arow * e.nKv + kvh) * e.gamma + gs) * hd;
        e.kb[off + d] = oa;
        e.kb[off + d + half] = ob;
        e.vb[off + d] = ya[u];
        e.vb[off + d + half] = yb[u];
      }
      if (j == 0) e.ssq[(int64_t)(head * hj + cp) * g.M + m] = ss;
    }
  }
}

// sublayer output y of 64 columns: store it and the row statistics the next
// GEMM's input norms are formed from (see NormIn)
template <int MT>
__device__ __forceinline__ void epi_sums(const GemmArgs& g, const EpiArgs& e, const f32x4* acc, int mbase, int cb, int n,
                         float* red) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, gq = lane >> 4;
  const float w1 = ld_act_v(e.w1, n, e.act_bf16);
  // residual loads issued together without a branch (a missing residual
  // reads Y's rows, same shape, and is zeroed after the loads)
  const float* hsrc = e.h ? e.h : e.Y;
  float hv[MT][4];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = min(mbase + t * 16 + 4 * gq + i, g.M - 1);
      hv[t][i] = hsrc[(int64_t)m * e.ldy + n];
    }
  if (!e.h)
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) hv[t][i] = 0.f;
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = mbase + t * 16 + 4 * gq + i;
      if (m < g.M) e.Y[(int64_t)m * e.ldy + n] = acc[t][i];
    }
  // fp64 products and sums (see RowStats)
  double* redd = (double*)red;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    // per lane: statistic q of row i at index 4 q + i; lane l of the row
    // group gets the 16 lanes' sum of index l
    double v[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const double y = acc[t][i], wy = (double)w1 * y, h = hv[t][i];
      v[i] = y * y;
      v[4 + i] = h * wy;
      v[8 + i] = wy * wy;
      v[12 + i] = h * h;
    }
    const double sum = row16_reduce_scatter(v);
    const int l = lane & 15;
    redd[((wave * MT * 16) + t * 16 + 4 * gq + (l & 3)) * 4 + (l >> 2)] = sum;
  }
  __syncthreads();
  for (int r = tid; r < MT * 16; r += 256) {
    const int m = mbase + r;
    if (m >= g.M) continue;
    RowStats s = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const double* p = redd + ((w * MT * 16) + r) * 4;
      s.x += p[0];
      s.y += p[1];
      s.z += p[2];
      s.w += p[3];
    }
    e.sums[(int64_t)cb * g.M + m] = s;
  }
}

// deepspec.ts, #computeLogits for one 64-entry vocabulary chunk:
// z = cap * tanh(y / cap), plus the chunk statistics the walk prunes with.
// For any previous token |markov_w2[v] . markov_w1[prev]| <= B_v :=
// ||w2_v|| * max ||w1||, so an entry with z_v + B_v below max_u (z_u - B_u)
// can never win a step.  Per (row, chunk): lo = max (z - B), hi = max (z + B).
template <int MT>
__device__ __forceinline__ void epi_lm(const GemmArgs& g, const EpiArgs& e, const f32x4* acc, int mbase, int cb, int n,
                       float* tile) {
  // (position within a set of four waves: an eight-wave workgroup runs two
  // column blocks, each set with its own tile)
  const int tid = threadIdx.x & 255, wave = tid >> 6, lane = tid & 63, gq = lane >> 4;
  const int V = g.N;
  const float b = e.aux ? walk_bound(e.aux, n, V) : 0.f;
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = t * 16 + 4 * gq + i, m = mbase + r;
      float z = acc[t][i];
      if (e.cap > 0.f) z = e.cap * tanh_fast(z / e.cap);
      if (e.smp.temperature > 0.f) {
        // sampling: the walk and its bounds see z + T g (base z to the logits)
        const int mr = min(m, g.M - 1), row = mr / e.smp.gamma;
        const float zs = z + e.smp.temperature * gumbel_noise(e.smp.seeds[row], mr - row * e.smp.gamma, n);
        if (m < g.M) {
          if (e.smp.zs != e.Y) e.Y[(int64_t)m * V + n] = z;
          e.smp.zs[(int64_t)m * V + n] = zs;
        }
        z = zs;
      } else if (m < g.M) {
        e.Y[(int64_t)m * V + n] = z;
      }
      // per 16-column tile: max over the tile's columns of z - b and z + b
      const float lo = row16_max(z - b), hi = row16_max(z + b);
      if ((lane & 15) == 0) {
        tile[(r * 4 + wave) * 2] = lo;
        tile[(r * 4 + wave) * 2 + 1] = hi;
      }
    }
  __syncthreads();
  for (int r = tid; r < MT * 16; r += 256) {
    const int m = mbase + r;
    if (m >= g.M) continue;
    float lo = tile[r * 8], hi = tile[r * 8 + 1];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      lo = fmaxf(lo, tile[(r * 4 + w) * 2]);
      hi = fmaxf(hi, tile[(r * 4 + w) * 2 + 1]);
    }
    e.lohi[(int64_t)m * e.NC + cb] = make_float2(lo, hi);
  }
}

// deepspec.ts, #geluTanhMlp: act = gelu_tanh(gate x) * up x.  Waves 0,1 (of
// each set of four) hold gate columns 32cb.., waves 2,3 the matching up
// columns; an eight-wave workgroup holds one tile per K half, added here.
template <int MT, int NW>
__device__ __forceinline__ void epi_gelu(const GemmArgs& g, const EpiArgs& e, const f32x4* acc, int mbase, int cb,
                                         float* ep, int half) {
  const int tid = threadIdx.x, wave = (tid & 255) >> 6, lane = tid & 63, gq = lane >> 4;
  constexpr int TILE = 4 * MT * 16 * 16;
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ep[half * TILE + (wave * MT * 16 + t * 16 + 4 * gq + i) * 16 + (lane & 15)] = acc[t][i];
  __syncthreads();
  for (int idx = tid; idx < MT * 16 * 32; idx += 64 * NW) {
    const int r = idx >> 5, col = idx & 31;
    const int m = mbase + r;
    if (m >= g.M) continue;
    const int og = ((col >> 4) * MT * 16 + r) * 16 + (col & 15);
    const int ou = ((2 + (col >> 4)) * MT * 16 + r) * 16 + (col & 15);
    float gt = ep[og], up = ep[ou];
    if (NW == 8) {
      gt += ep[TILE + og];
      up += ep[TILE + ou];
    }
    e.act[(int64_t)m * e.ld_act + 32 * cb + col] = gelu_tanh(gt) * up;
  }
}

// deepspec.ts, #projectContextKVRows for one (layer, kv head) and the rows
// [m0, m1) of the row block: V = rms(k) (no weight, no RoPE);
// K = RoPE(rms(k) * k_norm).  One wave per row; every load of a batch of
// rows is issued before the first use.
// SEP: a launch of its own (k_kv_epi): Y was written by an earlier kernel,
// so plain loads read it, and rinv is formed here while they are in flight.
template <int MT, int NT, bool SEP = false>
__device__ __forceinline__ void epi_kv(const GemmArgs& g, const EpiArgs& e, int m0, int m1, int grp,
                                       double* rinv, float2* rcs) {
  // one wave per four rows of the tile
  static_assert(MT * 16 == 4 * (NT / 64), "the K/V epilogue gives each wave four rows");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hd = e.hd, HJ = hd >> 6, half = hd >> 1;
  const int layer = grp / e.nKv, kvh = grp - layer * e.nKv;
  // per-layer pointers read once (a kernel-argument array indexed at run time)
  void* const kout = e.kout[layer];
  void* const vout = e.vout[layer];
  const void* const knw = e.kn_l[layer];
  const bool bf = e.act_bf16 != 0;
  // 1. loads: norm weights, then this wave's four rows of the group's y
  uint32_t kraw[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int d = min(lane + 64 * j, hd - 1);
    kraw[j] = *(const uint32_t*)((const char*)knw + (bf ? (d >> 1) * 4 : d * 4));
  }
  constexpr int RB = 4;
  const int mb = m0 + wave * RB;
  float y[RB][4];
#pragma unroll
  for (int rr = 0; rr < RB; ++rr) {
    const int m = min(mb + rr, m1 - 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = min(lane + 64 * j, hd - 1);
      y[rr][j] = SEP ? e.Y[(int64_t)m * g.N + grp * hd + d] : ld_coh(e.Y + (int64_t)m * g.N + grp * hd + d);
    }
  }
  // 2. while they are in flight: (cos, sin) of the tile's row positions and
  //    pairs.  The rows span batch rows b_first..b_last, whose starting
  //    positions are read with uniform (scalar) loads.
  if constexpr (SEP) {
    if (tid < half) rinv[tid] = rope_inv(tid, e.rope.step, e.rope.nrot);
    __syncthreads();
  }
  const int b_first = m0 / e.L, b_last = (m1 - 1) / e.L;
  for (int idx = tid; idx < MT * 16 * half; idx += NT) {
    const int r = idx / half, pr = idx - r * half;
    const int m = min(m0 + r, m1 - 1);
    const int b = m / e.L;
    int p0 = 0;
    for (int bb = b_first; bb <= b_last; ++bb) {
      const int pv = e.pos0[bb];  // uniform index: a scalar load, taken unconditionally
      p0 = b == bb ? pv : p0;
    }
    float c, sn;
    rope_cs_hw((int64_t)p0 + (m - b * e.L), rinv[pr], c, sn);
    rcs[idx] = make_float2(c, sn);
  }
  __syncthreads();
  float kw[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int d = lane + 64 * j;
    kw[j] = __uint_as_float(bf ? ((d & 1) ? (kraw[j] & 0xFFFF0000u) : (kraw[j] << 16)) : kraw[j]);
  }
  // 3. per row: RMS factor, V = y r, K = RoPE(y r k_norm)
#pragma unroll
  for (int rr = 0; rr < RB; ++rr) {
    const int m = mb + rr;  // wave-uniform
    if (m >= m1) break;
    const int b = m / e.L, i = m - b * e.L;
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j < HJ) ss += y[rr][j] * y[rr][j];
    const float r = rsqrtf(wave_sum(ss) / hd + e.eps);
    float t[4], kv[4], vv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) t[j] = y[rr][j] * r * kw[j];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = lane + 64 * j;
      float partner;
      if (HJ >= 2) partner = t[(j + HJ / 2) % HJ];
      else partner = __shfl_xor(t[0], 32);
      const float2 cs = rcs[(m - m0) * half + (d < half ? d : d - half)];
      vv[j] = y[rr][j] * r;
      kv[j] = d < half ? t[j] * cs.x - partner * cs.y : t[j] * cs.x + partner * cs.y;
    }
    const int64_t off = (((int64_t)b * e.nKv + kvh) * e.L + i) * hd;
    // (kout null: a V-only cache, K is rebuilt from V where it is read)
    if (bf) {
      uint16_t* const vo = (uint16_t*)vout + off;
      uint16_t* const ko = (uint16_t*)kout + off;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j < HJ) {
          vo[lane + 64 * j] = f2bf(vv[j]);
          if (kout) ko[lane + 64 * j] = f2bf(kv[j]);
        }
    } else {
      float* const vo = (float*)vout + off;
      float* const ko = (float*)kout + off;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j < HJ) {
          vo[lane + 64 * j] = vv[j];
          if (kout) ko[lane + 64 * j] = kv[j];
        }
    }
  }
}

// ---------------------------------------------------------------------------
// activation staging: items (row ml, 8 consecutive k) -> LDS hi / lo planes.
// stage_load issues the loads of one batch of XB items per thread into
// registers; stage_store converts them (norms for XM_NORM) and writes LDS.
// ---------------------------------------------------------------------------
// items per thread per batch, all of a 256-wide sub-slice where the
// registers allow: a 16-row tile has 2 per thread, a 32-row tile 4, a 64-row
// tile 8 (bf16 or f32 rows); normed 64-row tiles take batches of 4
template <int XM, int MT>
constexpr int xbatch() {
  return MT == 1 ? 2 : (MT == 2 || XM == XM_NORM ? 4 : 8);
}

template <int XB>
struct XRegs {
  f32x4 a[XB][2];  // XM_F32: x; XM_NORM: h
  f32x4 y[XB][2];  // XM_NORM: y
  u32x4 r16[XB];   // XM_BF16
};

// XM_NORM: the norm weights of the workgroup's K slice (at most KSMAX
// wide), eight per thread (threads below klen/8), go through LDS
// (wn[0..] = w1, wn[KSMAX..] = w2) instead of being loaded per item.
// Raw words: w[0], w[1] = w1, w[2], w[3] = w2.
constexpr int KSMAX = 2048;
__device__ __forceinline__ void normw_load(const GemmArgs& g, int kc, int klen, u32x4* w, int vt) {
  const NormIn& n = g.nin;
  const int k8 = min(vt, (klen >> 3) - 1);
  const bool bf = n.act_bf16 != 0;
  // unconditional loads from whichever vectors exist (at least one does)
  const void* p1 = n.y ? n.w1 : n.w2;
  const void* p2 = n.w2 ? n.w2 : p1;
  const Raw8 a = ld_act8(p1, kc + 8 * k8, bf), b = ld_act8(p2, kc + 8 * k8, bf);
  w[0] = a.a;
  w[1] = a.b;
  w[2] = b.a;
  w[3] = b.b;
}
__device__ __forceinline__ void normw_store(const GemmArgs& g, int klen, const u32x4* w, float* wn, int kcmax,
                                            int vt) {
  const NormIn& n = g.nin;
  const int k8 = vt;
  const bool bf = n.act_bf16 != 0;
  if (k8 < (klen >> 3)) {
    float v[8];
    Raw8 r;
    r.a = w[0];
    r.b = w[1];
    cvt_act8(r, bf, v);
    *(f32x4*)&wn[8 * k8] = f32x4{v[0], v[1], v[2], v[3]};
    *(f32x4*)&wn[8 * k8 + 4] = f32x4{v[4], v[5], v[6], v[7]};
    r.a = w[2];
    r.b = w[3];
    cvt_act8(r, bf, v);
    *(f32x4*)&wn[kcmax + 8 * k8] = f32x4{v[0], v[1], v[2], v[3]};
    *(f32x4*)&wn[kcmax + 8 * k8 + 4] = f32x4{v[4], v[5], v[6], v[7]};
  }
}

template <int XM, int MT>
__device__ __forceinline__ void stage_load(const GemmArgs& g, int mbase, int kc, int klen, int base,
                                           XRegs<xbatch<XM, MT>()>& r, int vt, bool live = true) {
  constexpr int XB = xbatch<XM, MT>();
  const int tid = vt;
  const int kq = klen >> 3;
  const int nitems = MT * 16 * kq;
#pragma unroll
  for (int b = 0; b < XB; ++b) {
    const int it = base + tid + 256 * b;
    const int ml = it / kq, k8 = it < nitems ? it - ml * kq : 0;
    // !live: the same number of loads, all of one row piece (a set of waves
    // that does not stage keeps its load count, so every wait stays exact)
    const int64_t m = live ? min(mbase + ml, g.M - 1) : 0;
    const int64_t k = live ? kc + 8 * k8 : 0;
    if constexpr (XM == XM_NORM) {
      // both loads always issued (from whichever of h, y exists) so the
      // number of loads in flight is fixed; stage_store ignores a missing one
      const NormIn& n = g.nin;
      const float* ph = n.h ? n.h : n.y;
      const float* py = n.y ? n.y : n.h;
      r.a[b][0] = *(const f32x4*)(ph + m * n.ld + k);
      r.a[b][1] = *(const f32x4*)(ph + m * n.ld + k + 4);
      r.y[b][0] = *(const f32x4*)(py + m * n.ld + k);
      r.y[b][1] = *(const f32x4*)(py + m * n.ld + k + 4);
    } else if constexpr (XM == XM_BF16) {
      r.r16[b] = *(const u32x4*)((const uint16_t*)g.X + m * g.ldx + k);
    } else {
      const float* px = (const float*)g.X + m * g.ldx + k;
      r.a[b][0] = *(const f32x4*)px;
      r.a[b][1] = *(const f32x4*)(px + 4);
    }
  }
}

// LDS position of staged 16-byte operand slot `slot` (16-slot groups hold one
// A-operand column of 16 rows): the low four bits are xor-ed with bits 4..7,
// so the staging stores (lanes along k, one row) spread over the banks
// instead of landing 256 bytes apart, while each MFMA operand read (lanes
// along the 16 rows of a group) stays a permutation within its group
__device__ __forceinline__ int xslot(int slot) { return slot ^ ((slot >> 4) & 15); }

template <int WK, int XM, int MT>
__device__ __forceinline__ void stage_store(const GemmArgs& g, int mbase, int kc, int klen, int base,
                                            const XRegs<xbatch<XM, MT>()>& r,
                                            u32x4* xhi, u32x4* xlo, float* xsum, int nfull, int ngmax,
                                            const float2* rs, const float* wn, int kcmax, bool write_h, int vt) {
  constexpr int XB = xbatch<XM, MT>();
  const int tid = vt;
  const int kq = klen >> 3;
  const int nitems = MT * 16 * kq;
#pragma unroll
  for (int b = 0; b < XB; ++b) {
    const int it = base + tid + 256 * b;
    if (it >= nitems) break;
    const int ml = it / kq, k8 = it - ml * kq;
    const int m = mbase + ml;
    const bool ok = m < g.M;
    float v[8];
    if constexpr (XM == XM_NORM) {
      const NormIn& n = g.nin;
      const float sc = rs[MT * 16].x;
      const float2 rr = rs[ml];
      const f32x4 w1a = *(const f32x4*)&wn[8 * k8], w1b = *(const f32x4*)&wn[8 * k8 + 4];
      const f32x4 w2a = *(const f32x4*)&wn[kcmax + 8 * k8], w2b = *(const f32x4*)&wn[kcmax + 8 * k8 + 4];
      float hn[8];
      if (n.h && n.y && n.w2) {
        // the backbone's sandwich (every operand present): hn = h sc + y (r1 sc w1),
        // x = hn (r2 w2); rows past M have r2 = 0 (norm_finish), so x = 0 there
        const float a1 = rr.x * sc;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float w1 = q < 4 ? w1a[q & 3] : w1b[q & 3], w2 = q < 4 ? w2a[q & 3] : w2b[q & 3];
          hn[q] = fmaf(r.y[b][q >> 2][q & 3], a1 * w1, r.a[b][q >> 2][q & 3] * sc);
          v[q] = hn[q] * (rr.y * w2);
        }
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float w1 = q < 4 ? w1a[q & 3] : w1b[q & 3], w2 = q < 4 ? w2a[q & 3] : w2b[q & 3];
          const float h = n.h ? r.a[b][q >> 2][q & 3] : 0.f;
          const float y = n.y ? r.y[b][q >> 2][q & 3] * rr.x * w1 : 0.f;
          hn[q] = (h + y) * sc;
          v[q] = ok ? (n.w2 ? hn[q] * rr.y * w2 : hn[q]) : 0.f;
        }
      }
      if (write_h && ok) {
        float* dst = n.hout + (int64_t)m * n.ld + kc + 8 * k8;
        *(f32x4*)dst = f32x4{hn[0], hn[1], hn[2], hn[3]};
        *(f32x4*)(dst + 4) = f32x4{hn[4], hn[5], hn[6], hn[7]};
      }
    } else if constexpr (XM == XM_BF16) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[2 * q] = ok ? __uint_as_float(r.r16[b][q] << 16) : 0.f;
        v[2 * q + 1] = ok ? __uint_as_float(r.r16[b][q] & 0xFFFF0000u) : 0.f;
      }
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = ok ? r.a[b][q >> 2][q & 3] : 0.f;
    }
    int s, qg;
    float e8[8];
    if constexpr (WK == WK_Q4) {
      const int grp = k8 >> 3, rr = k8 & 7;
      qg = rr >> 1;
      s = 2 * grp + (rr & 1);
      const int perm[8] = {0, 4, 1, 5, 2, 6, 3, 7};
      float sum = 0.f;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        e8[q] = v[perm[q]];
        sum += v[q];
      }
      atomicAdd(&xsum[ml * ngmax + grp], sum);
    } else {
      s = k8 >> 2;
      qg = k8 & 3;
#pragma unroll
      for (int q = 0; q < 8; ++q) e8[q] = v[q];
    }
    const int slot = ((ml >> 4) * nfull + s) * 64 + qg * 16 + (ml & 15);
    if constexpr (XM == XM_BF16) {
      xhi[xslot(slot)] = __builtin_bit_cast(u32x4, to_bf16x8(e8));
    } else {
      bf16x8 h, l;
      split8(e8, h, l);
      xhi[xslot(slot)] = __builtin_bit_cast(u32x4, h);
      xlo[xslot(slot)] = __builtin_bit_cast(u32x4, l);
    }
  }
}

// ---------------------------------------------------------------------------
// weights of one sub-slice in registers, and the MFMAs that consume them
// ---------------------------------------------------------------------------
template <int WK, int SMAX>
struct WRegs {
  u32x4 v[WK == WK_F32 ? 2 * SMAX : (WK == WK_BF16 ? SMAX : 1)];
  u32x2 q[WK == WK_Q4 ? SMAX / 2 : 1];
  float qs[WK == WK_Q4 ? SMAX / 2 : 1], qb[WK == WK_Q4 ? SMAX / 2 : 1];
};

template <int WK, int SMAX>
__device__ __forceinline__ void load_w(const GemmArgs& g, int si, int64_t wrow, int kc, int nsteps,
                                       WRegs<WK, SMAX>& w) {
  const int gq = (threadIdx.x & 63) >> 4;
  // every step is loaded (steps past nsteps repeat the last one and are not
  // used), so the number of loads in flight is fixed and the compiler's wait
  // counts stay exact
  if constexpr (WK == WK_BF16) {
    const uint16_t* p = (const uint16_t*)g.seg[si].w + wrow * g.K + kc + 8 * gq;
#pragma unroll
    for (int s = 0; s < SMAX; ++s) w.v[s] = *(const u32x4*)(p + 32 * min(s, nsteps - 1));
  } else if constexpr (WK == WK_F32) {
    const float* p = (const float*)g.seg[si].w + wrow * g.K + kc + 8 * gq;
#pragma unroll
    for (int s = 0; s < SMAX; ++s) {
      w.v[2 * s] = *(const u32x4*)(p + 32 * min(s, nsteps - 1));
      w.v[2 * s + 1] = *(const u32x4*)(p + 32 * min(s, nsteps - 1) + 4);
    }
  } else {
    const uint32_t* p = (const uint32_t*)g.seg[si].w;
    const uint16_t* ps = (const uint16_t*)g.seg[si].s;
    const uint16_t* pb = (const uint16_t*)g.seg[si].b;
#pragma unroll
    for (int j = 0; j < SMAX / 2; ++j)
      if (2 * j < nsteps) {
        const int64_t gi = q4_gemm_group(wrow, g.K, kc, j);
        w.q[j] = *(const u32x2*)(p + q4_gemm_word(wrow, g.K, kc, gq, j));
        w.qs[j] = bf2f(ps[gi]);
        w.qb[j] = bf2f(pb[gi]);
      }
  }
}

template <int WK, int XM, int MT, int SMAX>
__device__ __forceinline__ void mma_w(f32x4* acc, const WRegs<WK, SMAX>& w, const u32x4* xhi, const u32x4* xlo,
                                      const float* xsum, int nfull, int ngmax, int nsteps) {
  constexpr bool XBF = XM == XM_BF16;
  const int lane = threadIdx.x & 63, gq = lane >> 4;
  if constexpr (WK == WK_BF16) {
#pragma unroll
    for (int s = 0; s < SMAX; ++s)
      if (s < nsteps) {
        const bf16x8 wb = __builtin_bit_cast(bf16x8, w.v[s]);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const int o = xslot((t * nfull + s) * 64 + lane);
          acc[t] = mfma16(__builtin_bit_cast(bf16x8, xhi[o]), wb, acc[t]);
          if constexpr (!XBF) acc[t] = mfma16(__builtin_bit_cast(bf16x8, xlo[o]), wb, acc[t]);
        }
      }
  } else if constexpr (WK == WK_F32) {
#pragma unroll
    for (int s = 0; s < SMAX; ++s)
      if (s < nsteps) {
        float w8[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          w8[q] = __uint_as_float(w.v[2 * s][q]);
          w8[4 + q] = __uint_as_float(w.v[2 * s + 1][q]);
        }
        bf16x8 wh, wl;
        split8(w8, wh, wl);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const int o = xslot((t * nfull + s) * 64 + lane);
          const bf16x8 xh = __builtin_bit_cast(bf16x8, xhi[o]);
          acc[t] = mfma16(xh, wh, acc[t]);
          acc[t] = mfma16(xh, wl, acc[t]);
          if constexpr (!XBF) acc[t] = mfma16(__builtin_bit_cast(bf16x8, xlo[o]), wh, acc[t]);
        }
      }
  } else {
#pragma unroll
    for (int j = 0; j < SMAX / 2; ++j)
      if (2 * j < nsteps) {
        f32x4 tmp[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) tmp[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
          const bf16x8 wb = q4_decode(w.q[j][sub]);
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            const int o = xslot((t * nfull + 2 * j + sub) * 64 + lane);
            tmp[t] = mfma16(__builtin_bit_cast(bf16x8, xhi[o]), wb, tmp[t]);
            if constexpr (!XBF) tmp[t] = mfma16(__builtin_bit_cast(bf16x8, xlo[o]), wb, tmp[t]);
          }
        }
        const float sc = 16.f * w.qs[j], bc = w.qb[j] - sc;
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[t][i] += sc * tmp[t][i] + bc * xsum[(t * 16 + 4 * gq + i) * ngmax + j];
      }
  }
}

// LDS bytes of one staged activation sub-slice (hi / lo planes + q4 row sums)

// ---------------------------------------------------------------------------
// NW = 8 (unrolled, no split-K): eight waves, two per SIMD, as two sets of
// four with the same barriers.  gate|up: waves 4..7 run the same 64 columns
// over the second half of the K slice (their own staging buffers and row
// factors); the epilogue adds the two halves.  lm_head: waves 4..7 run the
// next 64 columns over the same K slice and multiply the activations the
// first set stages, so they are read once for 128 columns.  Two waves per
// SIMD hide one another's staging and MFMA phases behind the weight stream
// without the cross-workgroup reduction a split K would need.
template <int WK, int XM, int MT, int EPI, int NCH, int NW = 4, bool RM = false>
__global__ __launch_bounds__(64 * NW) void k_gemm(const GemmArgs g, const EpiArgs e) {
  static_assert(NW == 4 || (NW == 8 && NCH > 0 &&
                              ((MT == 1 && (EPI == EPI_GELU || EPI == EPI_LM)) || (MT == 2 && EPI == EPI_KV))),
                "eight waves: gate|up, lm_head or the 32-row context projection, unrolled");
  constexpr bool KH = NW == 8 && EPI != EPI_LM;     // sets split K
  constexpr bool COL2 = NW == 8 && EPI == EPI_LM;   // sets split columns
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int last_flag;
  __shared__ float2 rs_all[NW / 4][MT * 16 + 1];
  __shared__ __align__(16) float wn[XM == XM_NORM ? 2 * KSMAX : 1];
  // EPI_KV: 1 / wavelength of each RoPE pair (double), formed while the
  // first loads are in flight, and the (cos, sin) table of the tile's rows
  // built by whichever workgroup finishes a head group
  __shared__ double rinv[EPI == EPI_KV ? 128 : 1];
  __shared__ float2 rcs[EPI == EPI_KV ? MT * 16 * 128 : 1];
  // sub-slice width bound (the host plans kc <= KCMAX): 256 for one 16-row
  // tile, for the unrolled (double-buffered) variants and for fp32 weights,
  // else 512
  constexpr int KCMAX = (MT == 1 || NCH > 0 || WK == WK_F32) ? 256 : 512;
  constexpr int SMAX = KCMAX / 32;
  constexpr int XB = xbatch<XM, MT>();
  const int tid = threadIdx.x, lane = tid & 63, gq = lane >> 4;
  // position within the set of four waves, and which set
  const int vt = tid & 255, wave = vt >> 6, half = NW == 8 ? tid >> 8 : 0;
  const bool stager = !COL2 || half == 0;  // stages activations into LDS
  float2* const rs = rs_all[half];
  const int KC = NCH > 0 ? KCMAX : g.kc;  // unrolled variants run at KCMAX (the launcher checks)
  const int nfull = KC >> 5;
  const int ngmax = KC >> 6;
  const size_t xbuf = xbuf_bytes(WK, XM, MT, KC);

  // column block (pair), K slice and row block: RM (16-row tiles, several
  // row blocks) takes the XCD-aware order of stream_block_of, with
  // the grid sizes from the arguments (a run-time choice, or gridDim, puts a
  // scalar load ahead of the first weight address of every launch)
  static_assert(!RM || MT == 1, "the renumbered order is for 16-row tiles");
  int bx = blockIdx.x, by = blockIdx.y, bz = blockIdx.z;
  if constexpr (RM)
    stream_block_of(COL2 ? g.N >> 7 : g.N >> 6, (g.K + g.kslice - 1) / g.kslice, (g.M + 15) >> 4, blockIdx.x,
                    blockIdx.y, blockIdx.z, bx, by, bz);
  const int cb = COL2 ? 2 * bx + half : bx;
  // wave-uniform values in scalar registers, so that the weight segment is
  // read from the kernel arguments with scalar loads (a vector load of the
  // pointer would make the first weight load wait for every earlier load)
  const int n0w = __builtin_amdgcn_readfirstlane(wave_col<EPI>(cb, wave, g.N, e.hd));
  int si = 0;
  for (int i = 1; i < g.nseg; ++i)
    if (n0w >= g.seg[i].n0) si = i;
  si = __builtin_amdgcn_readfirstlane(si);
  const int64_t wrow = (int64_t)(n0w - g.seg[si].n0 + (lane & 15));
  const int mbase = bz * (MT * 16);
  const int kbeg = by * g.kslice;
  const int kend = min(g.K, kbeg + g.kslice);
  const bool write_h = XM == XM_NORM && g.nin.hout != nullptr && bx == 0;
  // NCH > 0: every slice is exactly NCH sub-slices of KC (fully unrolled,
  // so the loads of the next two sub-slices stay in flight with exact waits)
  const int nch = NCH > 0 ? NCH : (kend - kbeg + KC - 1) / KC;
  // this set's part of the slice (NW = 8: NCH sub-slices of each half)
  const int hbeg = KH ? kbeg + half * NCH * KC : kbeg;
  const int hlen = KH ? NCH * KC : kend - kbeg;

  f32x4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // 1. the small loads first (a wave's loads complete in order): row
  //    statistics and norm weights of the slice, then chunk 0's activations
  //    and weights (and chunk 1's, double-buffered, for a 16-row tile)
  RowStats nv[NV];
  float sc_in = 1.f;
  u32x4 wr[4];
  if constexpr (XM == XM_NORM) {
    norm_issue(g, mbase, nv, sc_in, vt);
    normw_load(g, hbeg, hlen, wr, vt);
  }
  XRegs<XB> xa, xb;
  WRegs<WK, SMAX> wa, wb;
  auto chunk_k = [&](int c) { return hbeg + c * KC; };
  auto chunk_len = [&](int c) { return NCH > 0 ? KC : min(KC, kend - chunk_k(c)); };
  stage_load<XM, MT>(g, mbase, chunk_k(0), chunk_len(0), 0, xa, vt, stager);
  load_w<WK, SMAX>(g, si, wrow, chunk_k(0), chunk_len(0) >> 5, wa);
  if (NCH > 1 || (MT == 1 && NCH == 0 && nch > 1)) {
    stage_load<XM, MT>(g, mbase, chunk_k(1), chunk_len(1), 0, xb, vt, stager);
    load_w<WK, SMAX>(g, si, wrow, chunk_k(1), chunk_len(1) >> 5, wb);
  }
  if constexpr (EPI == EPI_KV) {
    if (tid < (e.hd >> 1)) rinv[tid] = rope_inv(tid, e.rope.step, e.rope.nrot);
  }
  if constexpr (XM == XM_NORM) {
    norm_finish<MT>(g, mbase, nv, sc_in, rs, vt);
    if (stager) normw_store(g, hlen, wr, wn + (hbeg - kbeg), KSMAX, vt);
    __syncthreads();
  }

  // 2. per chunk: activations -> LDS buffer (hi / lo planes, A-operand
  //    order), then the MFMAs against the weight registers
  auto run_chunk = [&](int c, const XRegs<XB>& xr, const WRegs<WK, SMAX>& w, int buf) {
    const int kc = chunk_k(c), klen = chunk_len(c);
    u32x4* xhi = (u32x4*)(smem + (KH ? buf * 2 + half : buf) * xbuf);
    u32x4* xlo = xhi + MT * nfull * 64;
    float* xsum = (float*)((unsigned char*)xhi + xsum_offset(XM, MT, KC));
    if constexpr (WK == WK_Q4) {
      // each set of four waves clears its own buffer's sums (vt: thread within the set)
      for (int i = vt; i < MT * 16 * ngmax; i += 256) xsum[i] = 0.f;
      __syncthreads();
    }
    if (stager)
      stage_store<WK, XM, MT>(g, mbase, kc, klen, 0, xr, xhi, xlo, xsum, nfull, ngmax, rs, wn + (kc - kbeg), KSMAX,
                              write_h, vt);
    const int nitems = MT * 16 * (klen >> 3);
    for (int base = 256 * XB; base < nitems; base += 256 * XB) {
      XRegs<XB> xt;
      stage_load<XM, MT>(g, mbase, kc, klen, base, xt, vt, stager);
      if (stager)
        stage_store<WK, XM, MT>(g, mbase, kc, klen, base, xt, xhi, xlo, xsum, nfull, ngmax, rs, wn + (kc - kbeg),
                                KSMAX, write_h, vt);
    }
    __syncthreads();
    mma_w<WK, XM, MT, SMAX>(acc, w, xhi, xlo, xsum, nfull, ngmax, klen >> 5);
  };
  if constexpr (NCH > 0) {
#pragma unroll
    for (int c = 0; c < NCH; c += 2) {
      run_chunk(c, xa, wa, 0);
      if (c + 2 < NCH) {
        stage_load<XM, MT>(g, mbase, chunk_k(c + 2), KC, 0, xa, vt, stager);
        load_w<WK, SMAX>(g, si, wrow, chunk_k(c + 2), KC >> 5, wa);
      }
      if (c + 1 < NCH) {
        run_chunk(c + 1, xb, wb, 1);
        if (c + 3 < NCH) {
          stage_load<XM, MT>(g, mbase, chunk_k(c + 3), KC, 0, xb, vt, stager);
          load_w<WK, SMAX>(g, si, wrow, chunk_k(c + 3), KC >> 5, wb);
        }
      }
    }
  } else if constexpr (MT == 1) {
    // 16-row tile: two chunks in flight, two LDS buffers (a buffer is only
    // rewritten after the barrier that follows the other buffer's staging)
    for (int c = 0; c < nch; c += 2) {
      run_chunk(c, xa, wa, 0);
      if (c + 2 < nch) {
        stage_load<XM, MT>(g, mbase, chunk_k(c + 2), chunk_len(c + 2), 0, xa, vt);
        load_w<WK, SMAX>(g, si, wrow, chunk_k(c + 2), chunk_len(c + 2) >> 5, wa);
      }
      if (c + 1 < nch) {
        run_chunk(c + 1, xb, wb, 1);
        if (c + 3 < nch) {
          stage_load<XM, MT>(g, mbase, chunk_k(c + 3), chunk_len(c + 3), 0, xb, vt);
          load_w<WK, SMAX>(g, si, wrow, chunk_k(c + 3), chunk_len(c + 3) >> 5, wb);
        }
      }
    }
  } else {
    // 64-row tiles: one chunk at a time in one LDS buffer
    for (int c = 0; c < nch; ++c) {
      if (c > 0) {
        __syncthreads();
        stage_load<XM, MT>(g, mbase, chunk_k(c), chunk_len(c), 0, xa, vt);
        load_w<WK, SMAX>(g, si, wrow, chunk_k(c), chunk_len(c) >> 5, wa);
      }
      run_chunk(c, xa, wa, 0);
    }
  }
  __syncthreads();

  // 4. split-K reduction in the last workgroup of this column block
  const int S = gridDim.y;
  const int ncb = gridDim.x;
  const int n = n0w + (lane & 15);
  if (NW == 4 && S > 1) {
    // partials in accumulator order, P[s][tile][t][i][thread] with tile =
    // (row block, column block): every store and load instruction of a wave
    // covers 256 contiguous bytes
    const int64_t tiles = (int64_t)gridDim.z * ncb;
    const int64_t tile = (int64_t)bz * ncb + cb;
    auto pidx = [&](int sl, int t, int i) { return (((sl * tiles + tile) * MT + t) * 4 + i) * 256 + tid; };
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) st_coh(g.P + pidx(by, t, i), acc[t][i]);
    if (!arrive_last(e.cnt + bz * ncb + cb, S, &last_flag)) return;
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    constexpr int PB = MT == 1 ? 8 : 4;  // partial slices loaded per batch
    for (int s0 = 0; s0 < S; s0 += PB) {
      float part[PB][MT][4];
#pragma unroll
      for (int q = 0; q < PB; ++q)
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) part[q][t][i] = ld_coh(g.P + pidx(min(s0 + q, S - 1), t, i));
#pragma unroll
      for (int q = 0; q < PB; ++q)
        if (s0 + q < S)
#pragma unroll
          for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[t][i] += part[q][t][i];
    }
  }

  // 5. epilogue
  float* ep = (float*)smem;
  if constexpr (EPI == EPI_GELU) {
    epi_gelu<MT, NW>(g, e, acc, mbase, cb, ep, half);
  } else if constexpr (EPI == EPI_QK) {
    epi_qk<MT>(g, e, acc, mbase, cb, ep);
  } else if constexpr (EPI == EPI_SUMS) {
    epi_sums<MT>(g, e, acc, mbase, cb, n, ep);
  } else if constexpr (EPI == EPI_LM) {
    epi_lm<MT>(g, e, acc, mbase, cb, n, ep + half * 2 * 64 * MT);
  } else if constexpr (EPI == EPI_KV) {
    if constexpr (KH) {
      // add the second K half (waves 4..7) into the first through LDS
      if (half == 1)
#pragma unroll
        for (int t = 0; t < MT; ++t) *(f32x4*)&ep[(t * 256 + vt) * 4] = acc[t];
      __syncthreads();
      if (half == 0)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[t] += *(const f32x4*)&ep[(t * 256 + vt) * 4];
    }
    if (e.kv_defer) {
      // the separate epilogue launch reads Y after this kernel has ended
      if (half == 0)
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int m = mbase + t * 16 + 4 * gq + i;
            if (m < g.M) e.Y[(int64_t)m * g.N + n] = acc[t][i];
          }
      return;
    }
    if (half == 0)
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = mbase + t * 16 + 4 * gq + i;
          if (m < g.M) st_coh(e.Y + (int64_t)m * g.N + n, acc[t][i]);
        }
    const int gcols = e.group_cols;
    const int grp = (64 * cb) / gcols;
    const int ngroups = (g.N + gcols - 1) / gcols;
    const int members = (min(gcols, g.N - grp * gcols) + 63) / 64;
    if (!arrive_last(e.cnt + gridDim.z * ncb + bz * ngroups + grp, members, &last_flag)) return;
    epi_kv<MT, 64 * NW>(g, e, mbase, min(g.M, mbase + MT * 16), grp, rinv, rcs);
  }
}

// The epilogue of a GEMM whose product the tiled kernel (dspark_tall.hip)
// already wrote to T (row pitch ldt; S partial planes tstride apart, added
// here in slice order): one 16 x 64 tile per workgroup, the product read into
// the accumulator layout of the weight-streaming kernel (wave w: columns
// wave_col(cb, w) + lane mod 16, rows 4 (lane / 16) + i).
template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_epi(const GemmArgs g, const EpiArgs e, const float* T, int64_t ldt,
                                                  int S, int64_t tstride) {
  __shared__ __align__(16) float ep[4 * 16 * 16];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, gq = lane >> 4;
  const int cb = blockIdx.x, mbase = blockIdx.y * 16;
  const int n = wave_col<EPI>(cb, wave, g.N, e.hd) + (lane & 15);
  f32x4 acc[1];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[0][i] = T[(int64_t)min(mbase + 4 * gq + i, g.M - 1) * ldt + n];
  for (int s = 1; s < S; ++s) {
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = T[s * tstride + (int64_t)min(mbase + 4 * gq + i, g.M - 1) * ldt + n];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[0][i] += v[i];
  }
  if constexpr (EPI == EPI_GELU) epi_gelu<1, 4>(g, e, acc, mbase, cb, ep, 0);
  else if constexpr (EPI == EPI_QK) epi_qk<1>(g, e, acc, mbase, cb, ep);
  else if constexpr (EPI == EPI_SUMS) epi_sums<1>(g, e, acc, mbase, cb, n, ep);
  else if constexpr (EPI == EPI_LM) epi_lm<1>(g, e, acc, mbase, cb, n, ep);
}

// context K/V epilogue over a product already in e.Y (pitch N): one
// workgroup per (layer and kv-head group, 16 rows)
__global__ __launch_bounds__(256) void k_kv_epi(const GemmArgs g, const EpiArgs e) {
  __shared__ double rinv[128];
  __shared__ float2 rcs[16 * 128];
  const int mbase = blockIdx.y * 16;
  epi_kv<1, 256, true>(g, e, mbase, min(g.M, mbase + 16), blockIdx.x, rinv, rcs);
}

hipError_t launch_gemm_epi(const GemmArgs& a, const EpiArgs& e, int epi, const float* T, int64_t ldt, int S,
                           int64_t tstride, hipStream_t st) {
  const int mblocks = (a.M + 15) / 16;
  if (a.N % 64 != 0 || S < 1) return hipErrorInvalidValue;
  const dim3 grid(a.N / 64, mblocks);
  switch (epi) {
    case EPI_GELU: hipLaunchKernelGGL(k_gemm_epi<EPI_GELU>, grid, dim3(256), 0, st, a, e, T, ldt, S, tstride); break;
    case EPI_QK: hipLaunchKernelGGL(k_gemm_epi<EPI_QK>, grid, dim3(256), 0, st, a, e, T, ldt, S, tstride); break;
    case EPI_SUMS: hipLaunchKernelGGL(k_gemm_epi<EPI_SUMS>, grid, dim3(256), 0, st, a, e, T, ldt, S, tstride); break;
    case EPI_LM: hipLaunchKernelGGL(k_gemm_epi<EPI_LM>, grid, dim3(256), 0, st, a, e, T, ldt, S, tstride); break;
    case EPI_KV: {
      if (S != 1 || e.group_cols != e.hd || e.hd > 256 || a.N % e.hd != 0) return hipErrorInvalidValue;
      hipLaunchKernelGGL(k_kv_epi, dim3(a.N / e.hd, mblocks), dim3(256), 0, st, a, e);
      break;
    }
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

size_t gemm_lds_bytes(int wkind, int xmode, int mt, int kc) {
  const size_t b = xbuf_bytes(wkind, xmode, mt, kc) * (mt == 1 ? 2 : 1);  // a 16-row tile double-buffers
  const size_t tile = (size_t)mt * 16 * 64 * 4;                          // epilogue tiles
  return b > tile ? b : tile;
}

size_t gemm_counter_words(int M, int N, int mt, int group_cols) {
  const size_t mblocks = (M + mt * 16 - 1) / (mt * 16);
  const size_t ncb = N / 64;
  const size_t ngroups = group_cols > 0 ? (N + group_cols - 1) / group_cols : 0;
  return mblocks * (ncb + ngroups);
}

// input modes each epilogue is built for: the backbone GEMMs whose input is
// a normed residual (q|k, gate|up, lm_head) read XM_NORM; o and down read
// plain f32 rows; fc reads the target features (act dtype); k_proj reads the
// context rows (act dtype) or fc's output through hidden_norm.
template <int XM, int EPI>
constexpr bool built() {
  if constexpr (EPI == EPI_QK || EPI == EPI_GELU || EPI == EPI_LM) return XM == XM_NORM;
  if constexpr (EPI == EPI_SUMS) return XM != XM_NORM;
  return EPI == EPI_KV;
}

template <int WK, int XM, int MT, int EPI>
static hipError_t launch_one(const GemmArgs& a, const EpiArgs& e, int S, hipStream_t st) {
  if constexpr (built<XM, EPI>()) {
    const int mblocks = (a.M + MT * 16 - 1) / (MT * 16);
    const dim3 grid(a.N / 64, S, mblocks);
    size_t lds = gemm_lds_bytes(WK, XM, MT, a.kc);
    // unrolled variants (two sub-slices in flight, two LDS buffers) for bf16
    // weights with one 16-row tile, or 64-row tiles of bf16 rows, when every
    // slice is a whole number (1, 2, 4 or 8) of 256-wide sub-slices
    constexpr bool unrolled = WK == WK_BF16 && (MT <= 2 || XM == XM_BF16);
    int nch = 0;
    if (unrolled && a.kc == 256 && a.K % a.kslice == 0 && a.kslice % a.kc == 0) nch = a.kslice / a.kc;
    if (nch > 0) {
      const size_t two = xbuf_bytes(WK, XM, MT, 256) * 2;
      lds = two > lds ? two : lds;
    }
    if constexpr (MT == 2) {
      // 32-row tiles (context projection, bf16 rows): eight waves, the K
      // slice in two halves of 1, 2 or 4 sub-slices
      static_assert(WK == WK_BF16 && XM == XM_BF16 && EPI == EPI_KV, "32-row tiles: bf16 context projection");
      const int n2 = nch / 2;
      const size_t lds8 = xbuf_bytes(WK, XM, MT, 256) * 4;
      if (nch % 2 == 0) switch (n2) {
          case 1: hipLaunchKernelGGL((k_gemm<WK, XM, MT, EPI, 1, 8>), grid, dim3(512), lds8, st, a, e); return hipGetLastError();
          case 2: hipLaunchKernelGGL((k_gemm<WK, XM, MT, EPI, 2, 8>), grid, dim3(512), lds8, st, a, e); return hipGetLastError();
          case 4: hipLaunchKernelGGL((k_gemm<WK, XM, MT, EPI, 4, 8>), grid, dim3(512), lds8, st, a, e); return hipGetLastError();
          default: break;
        }
      return hipErrorInvalidValue;
    } else {
    // 16-row tiles: the XCD-aware block order (RM) over several row blocks
    auto sel = [&](auto rm) -> hipError_t {
    constexpr bool RM = decltype(rm)::value;
    if constexpr (unrolled && EPI == EPI_LM && MT == 1) {
      // lm_head over a whole row (no split-K): eight waves on two column
      // blocks that share one staging of the activations
      if (nch == 8 && S == 1 && (a.N / 64) % 2 == 0) {
        hipLaunchKernelGGL((k_gemm<WK, XM, MT, EPI, 8, 8, RM>), dim3(a.N / 128, S, grid.z), dim3(512), lds, st, a, e);
        return hipGetLastError();
      }
    }
    if constexpr (unrolled && EPI == EPI_GELU && MT == 1) {
      // gate|up over a whole row (no split-K): eight waves, four sub-slices
      // per K half, each half with its own two staging buffers
      if (nch == 8 && S == 1) {
        const size_t lds8 = xbuf_bytes(WK, XM, MT, 256) * 4;
        hipLaunchKernelGGL((k_gemm<WK, XM, MT, EPI, 4, 8, RM>), grid, dim3(512), lds8, st, a, e);
        return hipGetLastError();
      }
    }
    if constexpr (unrolled) {
      switch (nch) {
        case 1: hipLaunchKernelGGL((k_gemm<WK, XM, MT, EPI, 1, 4, RM>), grid, dim3(256), lds, st, a, e); return hipGetLastError();
        case 2: hipLaunchKernelGGL((k_gemm<WK, XM, MT, EPI, 2, 4, RM>), grid, dim3(256), lds, st, a, e); return hipGetLastError();
        case 4: hipLaunchKernelGGL((k_gemm<WK, XM, MT, EPI, 4, 4, RM>), grid, dim3(256), lds, st, a, e); return hipGetLastError();
        case 8: hipLaunchKernelGGL((k_gemm<WK, XM, MT, EPI, 8, 4, RM>), grid, dim3(256), lds, st, a, e); return hipGetLastError();
        default: break;
      }
    }
    hipLaunchKernelGGL((k_gemm<WK, XM, MT, EPI, 0, 4, RM>), grid, dim3(256), lds, st, a, e);
    return hipGetLastError();
    };
    if constexpr (MT == 1) {
      if (mblocks > 1) return sel(std::true_type{});
    }
    return sel(std::false_type{});
    }
  } else {
    return hipErrorInvalidValue;
  }
}

template <int WK, int XM, int MT>
static hipError_t launch_epi(const GemmArgs& a, const EpiArgs& e, int epi, int S, hipStream_t st) {
  switch (epi) {
    case EPI_QK: return launch_one<WK, XM, MT, EPI_QK>(a, e, S, st);
    case EPI_GELU: return launch_one<WK, XM, MT, EPI_GELU>(a, e, S, st);
    case EPI_SUMS: return launch_one<WK, XM, MT, EPI_SUMS>(a, e, S, st);
    case EPI_LM: return launch_one<WK, XM, MT, EPI_LM>(a, e, S, st);
    case EPI_KV: return launch_one<WK, XM, MT, EPI_KV>(a, e, S, st);
    default: return hipErrorInvalidValue;
  }
}

template <int WK, int XM>
static hipError_t launch_mt(const GemmArgs& a, const EpiArgs& e, int epi, int mt, int S, hipStream_t st) {
  if (mt == 1) return launch_epi<WK, XM, 1>(a, e, epi, S, st);
  if constexpr (WK == WK_BF16 && XM == XM_BF16) {
    if (mt == 2 && epi == EPI_KV) return launch_one<WK, XM, 2, EPI_KV>(a, e, S, st);
  }
  return hipErrorInvalidValue;
}

template <int WK>
static hipError_t launch_xm(const GemmArgs& a, const EpiArgs& e, int epi, int xmode, int mt, int S,
                            hipStream_t st) {
  if (xmode == XM_BF16) return launch_mt<WK, XM_BF16>(a, e, epi, mt, S, st);
  if (xmode == XM_NORM) return launch_mt<WK, XM_NORM>(a, e, epi, mt, S, st);
  return launch_mt<WK, XM_F32>(a, e, epi, mt, S, st);
}

hipError_t launch_gemm(const GemmArgs& a, const EpiArgs& e, int epi, int wkind, int xmode, int mt, int S,
                       hipStream_t st) {
  if (wkind == WK_BF16) return launch_xm<WK_BF16>(a, e, epi, xmode, mt, S, st);
  if (wkind == WK_F32) return launch_xm<WK_F32>(a, e, epi, xmode, mt, S, st);
  return launch_xm<WK_Q4>(a, e, epi, xmode, mt, S, st);
}

}  // namespace dsp
