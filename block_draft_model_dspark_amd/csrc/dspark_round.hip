// Row-wise kernels of the draft round: scaled embedding (with the RoPE table
// of the block positions), the split-softmax merge of the attention, and the
// Markov walk with its per-model bound data.  All arithmetic is fp32 (RoPE
// angles in fp64).
#include "dspark_kernels.hpp"
#include "dspark_common.hpp"

namespace dsp {

// embedding row of a table in f32 / bf16 / q4 storage, element k
__device__ __forceinline__ float table_elem(const void* E, const void* Es, const void* Eb, int kind, int group,
                                            int64_t row, int cols, int k) {
  if (kind == WK_F32) return ((const float*)E)[row * cols + k];
  if (kind == WK_BF16) return bf2f(((const uint16_t*)E)[row * cols + k]);
  const uint32_t w = ((const uint32_t*)E)[q4_word(row, cols, k)];
  const float q = (float)((w >> (4 * (k & 7))) & 0xFu);
  const int64_t gi = q4_group(row, cols, group, k);
  return bf2f(((const uint16_t*)Es)[gi]) * q + bf2f(((const uint16_t*)Eb)[gi]);
}

// ---------------------------------------------------------------------------
// deepspec.ts, #forwardBackbone: h = embed([anchor, MASK...]) * sqrt(H).
// Writes h, the row statistics (0, 0, 0, sum h^2) of every 64-column block
// that the first q|k GEMM forms layer 0's input norm from, the (cos, sin)
// table of the row's position for every RoPE pair, and the layer scalars.
// grid M, block 256.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_embed(const EmbedArgs a) {
  const int m = blockIdx.x, tid = threadIdx.x, M = gridDim.x;
  // the GEMM reduction counters of this round start at zero
  for (int i = m * 256 + tid; i < a.ncnt; i += gridDim.x * 256) a.cnt[i] = 0u;
  // residual scales as fp32 for the GEMMs' input norms
  if (m == 0 && tid <= a.nL) a.scal[tid] = tid == 0 ? 1.f : ld_act(a.scal_src[tid - 1], 0, a.act_bf16);
  const int row = m / a.rows.gamma, g = m - row * a.rows.gamma;
  const int64_t id = g == 0 ? a.rows.anchor[row] : a.mask_id;
  // the first eight bf16 values of this thread are loaded before the RoPE
  // table is formed, so the table's arithmetic overlaps the load
  u32x4 w_first = u32x4{0u, 0u, 0u, 0u};
  if (a.ekind == WK_BF16) w_first = *(const u32x4*)((const uint16_t*)a.E + id * a.H + min(8 * tid, a.H - 8));
  const int half = a.rope.hd >> 1;
  const int64_t pos = (int64_t)a.rows.pos[row] + g;
  for (int d = tid; d < half; d += 256) {
    float c, s;
    rope_cs_hw(pos, rope_inv(d, a.rope.step, a.rope.nrot), c, s);
    a.rt[(int64_t)m * half + d] = make_float2(c, s);
  }
  for (int k0 = 8 * tid; k0 < a.H; k0 += 2048) {
    float v[8];
    double ss = 0.0;
    if (a.ekind == WK_BF16) {
      // one 16-byte load of the eight bf16 values
      const u32x4 w = k0 == 8 * tid ? w_first : *(const u32x4*)((const uint16_t*)a.E + id * a.H + k0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[2 * q] = __uint_as_float(w[q] << 16);
        v[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = table_elem(a.E, a.Es, a.Eb, a.ekind, a.group, id, a.H, k0 + q);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      v[q] *= a.scale;
      ss += (double)v[q] * v[q];
    }
    float* dst = a.h + (int64_t)m * a.ldh + k0;
    *(f32x4*)dst = f32x4{v[0], v[1], v[2], v[3]};
    *(f32x4*)(dst + 4) = f32x4{v[4], v[5], v[6], v[7]};
    // eight threads per 64-column block
    ss += __shfl_xor(ss, 1);
    ss += __shfl_xor(ss, 2);
    ss += __shfl_xor(ss, 4);
    if ((tid & 7) == 0) a.sums[(int64_t)(k0 >> 6) * M + m] = RowStats{0.0, 0.0, 0.0, ss};
  }
}

// zero n words (the reduction counters of a context projection: its
// workspace may have held other data, e.g. a call of another shape).
// grid any, block 256.
__global__ __launch_bounds__(256) void k_zero(unsigned* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0u;
}

// ---------------------------------------------------------------------------
// split-softmax merge: O = sum_s e^{m_s - M} O_s / sum_s e^{m_s - M} l_s with
// M = max_s m_s; F16: the partials hold O_s / l_s in fp16 (weight e^{m_s-M} l_s).
// Each thread owns 8 head dims of one query row, so a split's partial is one
// 16-byte (fp16) or 32-byte (fp32) load per thread, eight splits in flight.
// fp32: dims 8c.. of the row, hd / 8 threads per row, grid
// ceil(A*nKv*nq / (256 / (hd / 8))).  fp16 (the attention's lane order
// [split, kvh, group of 16 rows, tile pair j, lane, 8]): thread (row group,
// j, lane) owns dims 32j + 4 (lane / 16) .. + 3 and the same + 16 of row
// 16 group + lane mod 16, so 64 threads read 1 KiB contiguous per split;
// grid A*nKv*ceil(nq/16)*(hd/32)*64 / 256.  block 256
// ---------------------------------------------------------------------------
constexpr int MERGE_SB = 8;          // splits loaded per batch
constexpr int MERGE_FEW_ROWS = 512;  // up to this many query rows: k_merge_rows

template <bool F16, bool LANE>
__global__ __launch_bounds__(256) void k_merge(const MergeArgs a) {
  const int tid = threadIdx.x;
  int j, kvh, row, d0, d1;  // query row, kv head, draft row; this thread's two runs of four dims
  int64_t pbase;            // fp16: halves offset of (split 0, kvh, group, pair, lane)
  const int ng = (a.nq + 15) / 16, np2 = a.hd / 32;
  if constexpr (F16 && LANE) {
    const int64_t gt = (int64_t)blockIdx.x * 256 + tid;
    const int lane = (int)(gt & 63);
    const int64_t rest = gt >> 6;  // ((row * nKv + kvh) * ng + group) * np2 + pair
    const int pair = (int)(rest % np2);
    const int64_t rg = rest / np2;  // (row * nKv + kvh) * ng + group
    const int grp = (int)(rg % ng);
    kvh = (int)((rg / ng) % a.nKv);
    row = (int)(rg / ((int64_t)ng * a.nKv));
    if (row >= a.A) return;
    j = grp * 16 + (lane & 15);
    if (j >= a.nq) return;
    d0 = 32 * pair + 4 * (lane >> 4);
    d1 = d0 + 16;
    pbase = (((int64_t)kvh * ng + grp) * np2 + pair) * 512 + 8 * lane;
  } else {
    const int lpq = a.hd >> 3;
    const int nrows = a.A * a.nKv * a.nq;
    const int qg = blockIdx.x * (256 / lpq) + tid / lpq;
    if (qg >= nrows) return;
    d0 = 8 * (tid - (tid / lpq) * lpq);
    d1 = d0 + 4;
    j = qg % a.nq;
    kvh = (qg / a.nq) % a.nKv;
    row = qg / (a.nq * a.nKv);
    pbase = 0;
  }
  const int s0 = a.split_off[row], ns = a.split_off[row + 1] - s0;
  const float2* ml = (const float2*)a.ml;
  auto mli = [&](int s) { return ((int64_t)(s0 + s) * a.nKv + kvh) * a.nq + j; };
  // running max over batches of MERGE_SB splits (all loads of a batch in
  // flight; a separate pass over the maxima would wait on each in turn)
  float mx = -INFINITY;
  float num[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, den = 0.f;
  for (int c0 = 0; c0 < ns; c0 += MERGE_SB) {
    u32x4 raw[MERGE_SB][F16 ? 1 : 2];
    float2 wv[MERGE_SB];
#pragma unroll
    for (int q = 0; q < MERGE_SB; ++q) {
      const int s = c0 + min(q, ns - c0 - 1);
      if constexpr (F16 && LANE) {
        // split stride: nKv * ng groups of 16 rows x hd halves
        raw[q][0] = *(const u32x4*)((const uint16_t*)a.opart + (int64_t)(s0 + s) * a.nKv * ng * 16 * a.hd + pbase);
      } else if constexpr (F16) {
        raw[q][0] = *(const u32x4*)((const uint16_t*)a.opart + mli(s) * a.hd + d0);
      } else {
        const int64_t i = mli(s) * a.hd + d0;
        raw[q][0] = *(const u32x4*)((const float*)a.opart + i);
        raw[q][1] = *(const u32x4*)((const float*)a.opart + i + 4);
      }
      wv[q] = ml[mli(s)];
    }
    float bm = mx;
#pragma unroll
    for (int q = 0; q < MERGE_SB; ++q) bm = fmaxf(bm, wv[q].x);  // repeats of the last split change nothing
    if (bm > mx) {
      const float r = expf(mx - bm);
#pragma unroll
      for (int e = 0; e < 8; ++e) num[e] *= r;
      den *= r;
      mx = bm;
    }
#pragma unroll
    for (int q = 0; q < MERGE_SB; ++q)
      if (c0 + q < ns) {
        const float w = expf(wv[q].x - mx), wl = w * wv[q].y;
        den += wl;
        float v[8];
        if constexpr (F16) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[2 * e] = f16_to_f32((uint16_t)(raw[q][0][e] & 0xFFFFu));
            v[2 * e + 1] = f16_to_f32((uint16_t)(raw[q][0][e] >> 16));
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[e] = __uint_as_float(raw[q][0][e]);
            v[4 + e] = __uint_as_float(raw[q][1][e]);
          }
        }
        const float ws = F16 ? wl : w;
#pragma unroll
        for (int e = 0; e < 8; ++e) num[e] += ws * v[e];
      }
  }
  const int rep = a.nH / a.nKv, hl = j / a.gamma, g = j - hl * a.gamma;
  const int h = kvh * rep + hl;
  const float rd = 1.f / den;
  const int64_t m = (int64_t)row * a.gamma + g;
  // dims d0.. (values 0..3) and d1.. (values 4..7)
  if (a.planes) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = num[e] * rd;
    bf16x8 hi, lo;
    split8(v, hi, lo);
    const u32x4 hw = __builtin_bit_cast(u32x4, hi), lw = __builtin_bit_cast(u32x4, lo);
    uint16_t* dst = a.planes + m * (a.nH * a.hd) + h * a.hd;
    *(u32x2*)(dst + d0) = u32x2{hw[0], hw[1]};
    *(u32x2*)(dst + d1) = u32x2{hw[2], hw[3]};
    *(u32x2*)(dst + a.plane + d0) = u32x2{lw[0], lw[1]};
    *(u32x2*)(dst + a.plane + d1) = u32x2{lw[2], lw[3]};
    return;
  }
  float* dst = a.O + m * a.ldo + h * a.hd;
  *(f32x4*)(dst + d0) = f32x4{num[0] * rd, num[1] * rd, num[2] * rd, num[3] * rd};
  *(f32x4*)(dst + d1) = f32x4{num[4] * rd, num[5] * rd, num[6] * rd, num[7] * rd};
}

// Few query rows with many splits each (a long context over few draft
// rows), fp16 partials in the wide attention's lane order: one workgroup of
// G waves per (draft row, kv head, group of 16 query rows, tile pair); wave w
// takes a contiguous share of the row's splits with k_merge's per-thread
// mapping (eight dims of one query row, one 16-byte load per split, 1 KiB
// contiguous per wave and split, MERGE_SB splits in flight), and the G
// waves' (max, sums) are merged in LDS by wave 0.  grid A*nKv*ceil(nq/16)*(hd/32)
template <int G>
__global__ __launch_bounds__(64 * G) void k_merge_split(const MergeArgs a) {
  __shared__ float sm[G][64], sden[G][64];
  __shared__ float snum[G][8][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ng = (a.nq + 15) / 16, np2 = a.hd / 32;
  const int64_t u = blockIdx.x;  // ((row * nKv + kvh) * ng + group) * np2 + pair
  const int pair = (int)(u % np2);
  const int64_t rg = u / np2;
  const int grp = (int)(rg % ng), kvh = (int)((rg / ng) % a.nKv), row = (int)(rg / ((int64_t)ng * a.nKv));
  const int j = grp * 16 + (lane & 15);
  const int jc = min(j, a.nq - 1);  // rows past nq compute on row nq - 1 and store nothing
  const int d0 = 32 * pair + 4 * (lane >> 4), d1 = d0 + 16;
  const int64_t pbase = (((int64_t)kvh * ng + grp) * np2 + pair) * 512 + 8 * lane;
  const int s0 = a.split_off[row], nsr = a.split_off[row + 1] - s0;
  const int per = (nsr + G - 1) / G, gs = wave * per, gn = max(0, min(per, nsr - gs));
  const float2* ml = (const float2*)a.ml;
  auto mli = [&](int s) { return ((int64_t)(s0 + s) * a.nKv + kvh) * a.nq + jc; };
  float mx = -INFINITY, den = 0.f;
  float num[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < gn; c0 += MERGE_SB) {  // (per wave: no barrier inside)
    u32x4 raw[MERGE_SB];
    float2 wv[MERGE_SB];
#pragma unroll
    for (int q = 0; q < MERGE_SB; ++q) {
      const int s = gs + c0 + min(q, gn - c0 - 1);
      raw[q] = *(const u32x4*)((const uint16_t*)a.opart + (int64_t)(s0 + s) * a.nKv * ng * 16 * a.hd + pbase);
      wv[q] = ml[mli(s)];
    }
    float bm = mx;
#pragma unroll
    for (int q = 0; q < MERGE_SB; ++q) bm = fmaxf(bm, wv[q].x);
    if (bm > mx) {
      const float r = expf(mx - bm);
#pragma unroll
      for (int e = 0; e < 8; ++e) num[e] *= r;
      den *= r;
      mx = bm;
    }
#pragma unroll
    for (int q = 0; q < MERGE_SB; ++q)
      if (c0 + q < gn) {
        const float wl = expf(wv[q].x - mx) * wv[q].y;
        den += wl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          num[2 * e] += wl * f16_to_f32((uint16_t)(raw[q][e] & 0xFFFFu));
          num[2 * e + 1] += wl * f16_to_f32((uint16_t)(raw[q][e] >> 16));
        }
      }
  }
  sm[wave][lane] = mx;
  sden[wave][lane] = den;
#pragma unroll
  for (int e = 0; e < 8; ++e) snum[wave][e][lane] = num[e];
  __syncthreads();
  if (wave != 0 || j >= a.nq) return;
  // wave 0 always holds splits (per >= 1), so the common reference is finite
  float M = sm[0][lane];
#pragma unroll
  for (int w = 1; w < G; ++w) M = fmaxf(M, sm[w][lane]);
  den = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) num[e] = 0.f;
#pragma unroll
  for (int w = 0; w < G; ++w)
    if (sm[w][lane] != -INFINITY) {
      const float f = expf(sm[w][lane] - M);
      den += sden[w][lane] * f;
#pragma unroll
      for (int e = 0; e < 8; ++e) num[e] += snum[w][e][lane] * f;
    }
  const int rep = a.nH / a.nKv, hl = j / a.gamma, g = j - hl * a.gamma;
  const int h = kvh * rep + hl;
  const float rd = 1.f / den;
  const int64_t m = (int64_t)row * a.gamma + g;
  // dims d0.. (values 0..3) and d1.. (values 4..7)
  if (a.planes) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = num[e] * rd;
    bf16x8 hi, lo;
    split8(v, hi, lo);
    const u32x4 hw = __builtin_bit_cast(u32x4, hi), lw = __builtin_bit_cast(u32x4, lo);
    uint16_t* dst = a.planes + m * (a.nH * a.hd) + h * a.hd;
    *(u32x2*)(dst + d0) = u32x2{hw[0], hw[1]};
    *(u32x2*)(dst + d1) = u32x2{hw[2], hw[3]};
    *(u32x2*)(dst + a.plane + d0) = u32x2{lw[0], lw[1]};
    *(u32x2*)(dst + a.plane + d1) = u32x2{lw[2], lw[3]};
    return;
  }
  float* dst = a.O + m * a.ldo + h * a.hd;
  *(f32x4*)(dst + d0) = f32x4{num[0] * rd, num[1] * rd, num[2] * rd, num[3] * rd};
  *(f32x4*)(dst + d1) = f32x4{num[4] * rd, num[5] * rd, num[6] * rd, num[7] * rd};
}

// Few query rows (a single draft row): one workgroup per query row, one
// thread per head dim, the splits in passes of MERGE_RB with every partial
// load of a pass in flight.  grid A*nKv*nq, block hd (>= 64)
constexpr int MERGE_RB = 32;

template <bool F16, bool LANE>
__global__ __launch_bounds__(256) void k_merge_rows(const MergeArgs a) {
  __shared__ float2 wl[MERGE_RB];
  __shared__ float cmax;
  const int idx = blockIdx.x, tid = threadIdx.x;
  const int j = idx % a.nq, kvh = (idx / a.nq) % a.nKv, row = idx / (a.nq * a.nKv);
  const int s0 = a.split_off[row], ns = a.split_off[row + 1] - s0;
  const float2* ml = (const float2*)a.ml;
  // fp16 lane order: thread tid reads half (tid mod 8) of lane j mod 16 +
  // 16 ((tid mod 32) / 8) in tile pair tid / 32 (eight threads per 16-byte
  // piece), which is dim 16 (2 pair + half / 4) + 4 ((tid mod 32) / 8) + half mod 4
  const int pr = tid >> 5, gq8 = (tid & 31) >> 3, hv = tid & 7;
  const int dim = F16 && LANE ? 16 * (2 * pr + (hv >> 2)) + 4 * gq8 + (hv & 3) : tid;
  const int ng = (a.nq + 15) / 16;
  float num = 0.f, den = 0.f, mrun = -INFINITY;
  for (int c0 = 0; c0 < ns; c0 += MERGE_RB) {
    const int cn = min(MERGE_RB, ns - c0);
    float o[MERGE_RB];
#pragma unroll
    for (int q = 0; q < MERGE_RB; ++q) {
      const int s = s0 + c0 + min(q, cn - 1);
      if constexpr (F16 && LANE) {
        const int64_t i = ((((int64_t)s * a.nKv + kvh) * ng + j / 16) * (a.hd / 32) + pr) * 512 +
                          8 * ((j & 15) + 16 * gq8) + hv;
        o[q] = f16_to_f32(((const uint16_t*)a.opart)[i]);
      } else if constexpr (F16) {
        o[q] = f16_to_f32(((const uint16_t*)a.opart)[(((int64_t)s * a.nKv + kvh) * a.nq + j) * a.hd + tid]);
      } else {
        o[q] = ((const float*)a.opart)[(((int64_t)s * a.nKv + kvh) * a.nq + j) * a.hd + tid];
      }
    }
    const float2 v = ml[((int64_t)(s0 + c0 + min(tid, cn - 1)) * a.nKv + kvh) * a.nq + j];
    if (tid < 64) {
      const float mm = wave_max(tid < cn ? v.x : -INFINITY);
      if (tid == 0) cmax = mm;
    }
    __syncthreads();
    const float mnew = fmaxf(mrun, cmax);
    if (tid < cn) {
      const float w = expf(v.x - mnew);
      wl[tid] = make_float2(w, w * v.y);
    }
    const float rescale = expf(mrun - mnew);
    num *= rescale;
    den *= rescale;
    mrun = mnew;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < MERGE_RB; ++q)
      if (q < cn) {
        num += (F16 ? wl[q].y : wl[q].x) * o[q];
        den += wl[q].y;
      }
    __syncthreads();
  }
  const int rep = a.nH / a.nKv, hl = j / a.gamma, g = j - hl * a.gamma;
  const int h = kvh * rep + hl;
  const int64_t m = (int64_t)row * a.gamma + g;
  const float x = num / den;
  if (a.planes) {
    const __bf16 hi = (__bf16)x;
    const __bf16 lo = (__bf16)(x - (float)hi);
    a.planes[m * (a.nH * a.hd) + h * a.hd + dim] = __builtin_bit_cast(uint16_t, hi);
    a.planes[a.plane + m * (a.nH * a.hd) + h * a.hd + dim] = __builtin_bit_cast(uint16_t, lo);
    return;
  }
  a.O[m * a.ldo + h * a.hd + dim] = x;
}

// markov_w1 / markov_w2 element (table_elem with the head's own storage)
__device__ __forceinline__ float head_elem(const void* w, const void* s, const void* b, int kind, int group,
                                           int64_t row, int cols, int k) {
  return table_elem(w, s, b, kind, group, row, cols, k);
}

// ---------------------------------------------------------------------------
// deepspec.ts, draftRows sequential walk at temperature 0:
//   prev = anchor; for k < gamma: tok = argmax(z[k] + markov_w2 markov_w1[prev]); prev = tok
// One workgroup per draft row; ties go to the lower vocabulary index.
//
// Only entries that survive the bound test of the logits epilogue can win a
// step (the winner w has z_w + B_w >= u_w >= max_v (z_v - B_v)), and that set
// C_k does not depend on the previous token.  The previous token of step k
// is the winner of step k-1, so it lies in C_{k-1} (the anchor for k = 0).
// The fast path therefore builds every C_k from the per-chunk bounds and the
// logits of the chunks that can hold a member, scores the table
// z_k[c] + w2[c] . w1[p] for p in C_{k-1}, c in C_k in parallel, then walks
// the table in LDS.  If some step keeps more than WALK_CMAX entries or too
// many chunks pass, the row takes the per-step path that scores every
// surviving entry against the actual previous token.
// grid A, block WALK_NT
// ---------------------------------------------------------------------------
constexpr int WALK_CMAX = 16;   // fast-path candidates per step
constexpr int WALK_GMAX = 32;   // block size bound
constexpr int WALK_FMAX = 512;  // fast-path flagged (step, chunk) pairs per row
constexpr int WALK_TPT = 8;     // threads per scored (prev, candidate) pair
constexpr int WALK_NT = 1024;   // threads per row

// dot(markov_w2[v], e) for a row of `rank` entries
__device__ __forceinline__ float w2_dot(const WalkArgs& a, int64_t v, const float* e) {
  float dot = 0.f;
  if (a.wkind == WK_BF16) {
    const u32x4* p = (const u32x4*)((const uint16_t*)a.w2 + v * a.rank);
    for (int j8 = 0; j8 < (a.rank >> 3); ++j8) {
      const u32x4 w = p[j8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        dot += __uint_as_float(w[q] << 16) * e[8 * j8 + 2 * q];
        dot += __uint_as_float(w[q] & 0xFFFF0000u) * e[8 * j8 + 2 * q + 1];
      }
    }
  } else {
    for (int j = 0; j < a.rank; ++j) dot += head_elem(a.w2, a.w2s, a.w2b, a.wkind, a.group, v, a.rank, j) * e[j];
  }
  return dot;
}

// part `sub` of markov_w2[v] . markov_w1[prev]: 8-entry groups sub, sub + TPT, ...
__device__ __forceinline__ float w1w2_dot_part(const WalkArgs& a, int64_t prev, int64_t v, int sub) {
  const int n8 = a.rank >> 3;
  float dot = 0.f;
  if (a.wkind == WK_BF16) {
    const u32x4* p1 = (const u32x4*)((const uint16_t*)a.w1 + prev * a.rank);
    const u32x4* p2 = (const u32x4*)((const uint16_t*)a.w2 + v * a.rank);
    for (int j0 = sub; j0 < n8; j0 += 4 * WALK_TPT) {
      u32x4 x1[4], x2[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = min(j0 + q * WALK_TPT, n8 - 1);
        x1[q] = p1[j];
        x2[q] = p2[j];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (j0 + q * WALK_TPT < n8)
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            dot += __uint_as_float(x1[q][h] << 16) * __uint_as_float(x2[q][h] << 16);
            dot += __uint_as_float(x1[q][h] & 0xFFFF0000u) * __uint_as_float(x2[q][h] & 0xFFFF0000u);
          }
    }
  } else {
    for (int j8 = sub; j8 < n8; j8 += WALK_TPT)
      for (int j = 8 * j8; j < 8 * j8 + 8; ++j)
        dot += head_elem(a.w1, a.w1s, a.w1b, a.wkind, a.group, prev, a.rank, j) *
               head_elem(a.w2, a.w2s, a.w2b, a.wkind, a.group, v, a.rank, j);
  }
  return dot;
}

// The per-step path: each step scores every entry that can still win against
// the actual previous token (vanilla head: e = markov_w1[prev]) or the state
// the previous tokens drove (RNN head: e = s_k).  With n = ||e|| the bias of
// entry v is at most n ||markov_w2[v]|| = t B_v, t = n / (the model-wide
// bound of ||e|| that B uses) <= 1, and over a chunk
// z_v + t B_v <= ((1 + t) hi + (1 - t) lo) / 2 by the epilogue's statistics.
// The exact best score of the chunk with the largest such bound is a
// threshold; the chunks whose bound reaches it are scored one wave per
// chunk, one lane per entry.
__device__ void walk_per_step(const WalkArgs& a, int row) {
  __shared__ float redu[WALK_NT / 64];
  __shared__ int redi[WALK_NT / 64];
  __shared__ float e[256];
  __shared__ float st[256];         // RNN head: s_{k-1}
  __shared__ float part[WALK_NT];   // RNN head: partial sums of s_{k-1} wh
  __shared__ int clist[WALK_NT];    // chunks to score
  __shared__ int ncl, prev_s;
  __shared__ float thr_s;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, G = a.rows.gamma, r = a.rank, NC = a.NC;
  const bool rnn = a.rnn && r > 0;
  if (tid == 0) prev_s = a.rows.anchor[row];
  if (rnn)
    for (int j = tid; j < r; j += WALK_NT) st[j] = 0.f;
  __syncthreads();
  const float nb = a.aux ? a.aux[a.V] : 0.f;
  for (int k = 0; k < G; ++k) {
    const int64_t m = (int64_t)row * G + k;
    const float2* lh = a.lohi + m * NC;
    const int prev = prev_s;
    if (rnn) {
      // s_k = tanh(s_{k-1} wh + w1[prev] + bh): entry j is column j of s wh,
      // its sum split over P groups of rows
      const int P = min(WALK_NT / r, r), j = tid % r, p = tid / r;
      if (p < P) {
        float acc = 0.f;
        for (int i = p; i < r; i += P) acc += st[i] * head_elem(a.wh, a.whs, a.whb, a.wkind, a.group, i, r, j);
        part[p * r + j] = acc;
      }
      __syncthreads();
      if (tid < r) {
        float acc = ld_act(a.bh, tid, a.act_bf16) + head_elem(a.w1, a.w1s, a.w1b, a.wkind, a.group, prev, r, tid);
        for (int q = 0; q < P; ++q) acc += part[q * r + tid];
        const float s = tanhf(acc);
        e[tid] = s;
        st[tid] = s;
      }
    } else if (tid < r) {
      e[tid] = head_elem(a.w1, a.w1s, a.w1b, a.wkind, a.group, prev, r, tid);
    }
    // t from ||e|| (a relative margin for its rounding; t <= 1 always holds
    // mathematically, the clamp only absorbs that margin)
    const float n2 = block_sum(tid < r ? e[tid] * e[tid] : 0.f, redu);
    const float t = nb > 0.f ? fminf(1.f, sqrtf(n2) * (1.f + 1e-4f) / nb) : 0.f;
    const float wt = 0.5f * (1.f + t), wl = 0.5f * (1.f - t);
    // seed chunk: the largest bound
    float bu = -INFINITY;
    int bi = 0x7fffffff;
    for (int c = tid; c < NC; c += WALK_NT) {
      const float2 q = lh[c];
      const float ub = wt * q.y + wl * q.x;
      if (better(ub, c, bu, bi)) {
        bu = ub;
        bi = c;
      }
    }
    block_argmax(bu, bi, redu, redi);
    if (wave == 0) {
      const int v = (bi >= 0 && bi < NC ? bi : 0) * WALK_CHUNK + lane;
      float u = -INFINITY;
      if (v < a.V) {
        u = a.z[m * a.V + v];
        if (r > 0) u += w2_dot(a, v, e);
      }
      u = wave_max(u);
      if (lane == 0) {
        float th = u - 1e-4f * (1.f + fabsf(u));
        if (!(th > -INFINITY)) th = -INFINITY;  // non-finite seed scores: keep every finite entry
        thr_s = th;
        ncl = 0;
      }
    }
    __syncthreads();
    const float thr = thr_s;
    float wu = -INFINITY;
    int wi = 0x7fffffff;
    for (int c0 = 0; c0 < NC; c0 += WALK_NT) {
      const int c = c0 + tid;
      if (c < NC) {
        const float2 q = lh[c];
        if (wt * q.y + wl * q.x >= thr) clist[atomicAdd(&ncl, 1)] = c;
      }
      __syncthreads();
      const int nl = ncl;
      for (int l = wave; l < nl; l += WALK_NT / 64) {
        const int v = clist[l] * WALK_CHUNK + lane;
        if (v < a.V) {
          const float zv = a.z[m * a.V + v];
          if (zv + t * (a.aux ? walk_bound(a.aux, v, a.V) : 0.f) >= thr) {
            const float u = r > 0 ? zv + w2_dot(a, v, e) : zv;
            if (better(u, v, wu, wi)) {
              wu = u;
              wi = v;
            }
          }
        }
      }
      if (c0 + WALK_NT < NC) {
        __syncthreads();
        if (tid == 0) ncl = 0;
        __syncthreads();
      }
    }
    block_argmax(wu, wi, redu, redi);
    if (tid == 0) {
      // no finite candidate (non-finite logits): report -1 and keep a valid row index
      const bool ok = wi >= 0 && wi < a.V;
      a.tokens[m] = ok ? wi : -1;
      prev_s = ok ? wi : 0;
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(WALK_NT) void k_walk(const WalkArgs a) {
  __shared__ int cand[WALK_GMAX][WALK_CMAX];
  __shared__ float candz[WALK_GMAX][WALK_CMAX];  // the candidates' logits
  __shared__ int ncand[WALK_GMAX];
  __shared__ int best[WALK_GMAX][WALK_CMAX];     // [k][prev index]: index of the step-k winner
  __shared__ float thr[WALK_GMAX];
  __shared__ float tab[WALK_GMAX][WALK_CMAX][WALK_CMAX];  // [k][prev index][candidate index]
  __shared__ int flag_kc[WALK_FMAX];                      // k << 24 | chunk
  __shared__ int toff[WALK_GMAX + 1];
  __shared__ int nflag, slow;
  const int row = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, G = a.rows.gamma;
  const int NC = a.NC;
  if (a.rnn) {
    // the RNN head's bias depends on the whole prefix, not only on the
    // previous token: no per-(step, previous candidate) table
    walk_per_step(a, row);
    return;
  }
  if (tid < WALK_GMAX) ncand[tid] = 0;
  if (tid == 0) {
    nflag = 0;
    slow = 0;
  }
  // 1. per-step threshold max_c lo_c: TPS threads per step, 16 chunk
  //    statistics in flight each (kept for step 2 when one batch covers them)
  int TPS = 64;  // a power of two within one wave
  while (TPS * G > WALK_NT) TPS >>= 1;
  const int k = tid / TPS, sub = tid - k * TPS;
  const bool kok = k < G;
  const float2* lh = a.lohi + ((int64_t)row * G + min(k, G - 1)) * NC;
  float lm = -INFINITY;
  float2 v[16];
  for (int c0 = 0; c0 < NC; c0 += TPS * 16) {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = lh[min(c0 + sub + TPS * i, NC - 1)];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (c0 + sub + TPS * i < NC) lm = fmaxf(lm, v[i].x);
  }
  for (int o = TPS >> 1; o > 0; o >>= 1) lm = fmaxf(lm, __shfl_xor(lm, o));
  const float th = lm - 1e-4f * (1.f + fabsf(lm));
  if (kok && sub == 0) thr[k] = th;
  __syncthreads();
  // 2. chunks whose best z + B reaches the threshold
  for (int c0 = 0; c0 < NC; c0 += TPS * 16) {
    if (NC > TPS * 16) {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = lh[min(c0 + sub + TPS * i, NC - 1)];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int c = c0 + sub + TPS * i;
      if (kok && c < NC && v[i].y >= th) {
        const int f = atomicAdd(&nflag, 1);
        if (f < WALK_FMAX) flag_kc[f] = (k << 24) | c;
      }
    }
  }
  __syncthreads();
  const int nf = nflag;
  if (nf > WALK_FMAX) slow = 1;
  // 3. candidates: the entries of the passing chunks that reach the
  //    threshold; one wave per chunk, four chunks in flight per wave
  const int nfm = min(nf, WALK_FMAX);
  for (int f0 = wave * 4; f0 < nfm; f0 += 4 * (WALK_NT / 64)) {
    float zz[4], bb[4];
    int kq[4], vq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int f = flag_kc[min(f0 + q, nfm - 1)];
      kq[q] = f >> 24;
      vq[q] = (f & 0xFFFFFF) * WALK_CHUNK + lane;
      zz[q] = a.z[((int64_t)row * G + kq[q]) * a.V + vq[q]];
      bb[q] = a.aux ? walk_bound(a.aux, vq[q], a.V) : 0.f;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (f0 + q >= nfm) break;
      const bool pass = zz[q] + bb[q] >= thr[kq[q]];
      const uint64_t bal = __ballot(pass);
      const int cnt = __popcll(bal);
      if (cnt == 0) continue;
      int base = 0;
      if (lane == 0) base = atomicAdd(&ncand[kq[q]], cnt);
      base = __shfl(base, 0);
      if (base + cnt > WALK_CMAX) {
        if (lane == 0) slow = 1;
      } else if (pass) {
        const int ci = base + __popcll(bal & ((1ull << lane) - 1ull));
        cand[kq[q]][ci] = vq[q];
        candz[kq[q]][ci] = zz[q];
      }
    }
  }
  __syncthreads();
  if (slow) {
    walk_per_step(a, row);
    return;
  }
  // 4. score table: pairs (p, c) of every step, WALK_TPT threads per pair
  if (tid == 0) {
    int o = 0;
    for (int kk = 0; kk < G; ++kk) {
      toff[kk] = o;
      o += (kk == 0 ? 1 : ncand[kk - 1]) * ncand[kk];
    }
    toff[G] = o;
  }
  __syncthreads();
  const int ntri = toff[G];
  for (int t0 = 0; t0 < ntri; t0 += WALK_NT / WALK_TPT) {
    const int t = t0 + tid / WALK_TPT, ts = tid % WALK_TPT;
    const bool ok = t < ntri;
    int kk = 0, pi = 0, ci = 0, prev = 0, v = 0;
    if (ok) {
      while (toff[kk + 1] <= t) ++kk;
      const int r = t - toff[kk], nc = ncand[kk];
      pi = r / nc;
      ci = r - pi * nc;
      prev = kk == 0 ? a.rows.anchor[row] : cand[kk - 1][pi];
      v = cand[kk][ci];
    }
    float dot = (ok && a.rank > 0) ? w1w2_dot_part(a, prev, v, ts) : 0.f;
#pragma unroll
    for (int o = WALK_TPT >> 1; o > 0; o >>= 1) dot += __shfl_xor(dot, o);
    if (ok && ts == 0) tab[kk][pi][ci] = candz[kk][ci] + dot;
  }
  __syncthreads();
  // 5. for every step and previous candidate, the winning candidate (all in
  //    parallel: one thread per (k, prev index), ties to the lower id)
  for (int t = tid; t < G * WALK_CMAX; t += WALK_NT) {
    const int kk = t / WALK_CMAX, pi = t - kk * WALK_CMAX;
    const int np = kk == 0 ? 1 : ncand[kk - 1], nc = ncand[kk];
    int bi = 0;
    if (pi < np && nc > 0) {
      float bu = tab[kk][pi][0];
      int bv = cand[kk][0];
      for (int ci = 1; ci < nc; ++ci) {
        const float u = tab[kk][pi][ci];
        const int v = cand[kk][ci];
        if (better(u, v, bu, bv)) {
          bu = u;
          bv = v;
          bi = ci;
        }
      }
    }
    best[kk][pi] = nc > 0 ? bi : -1;
  }
  __syncthreads();
  // 6. the walk itself: a chain of lookups best[k][prev index]
  if (tid == 0) {
    int pi = 0;
    for (int kk = 0; kk < G; ++kk) {
      const int bi = best[kk][pi];
      a.tokens[(int64_t)row * G + kk] = bi >= 0 ? cand[kk][bi] : -1;
      pi = bi >= 0 ? bi : 0;
    }
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
  // |markov_w2[v] . x| <= ||markov_w2[v]|| ||x||; x = markov_w1[prev] (vanilla
  // head) or the RNN state, whose entries are tanh values (||s|| <= sqrt(rank))
  const float xb = a.rnn ? sqrtf((float)a.rank) : sqrtf(s1);
  if (l == 0) {
    a.aux[v] = sqrtf(s2) * (1.f + 1e-5f);
    atomicMax((unsigned int*)&a.aux[a.V], __float_as_uint(xb * (1.f + 1e-5f)));
  }
}

// ---------------------------------------------------------------------------
// deepspec.ts, #confidence and the draftRows truncation rule
// (_confident_prefix_length):
//   c_k = sigmoid(proj . [x_k ; markov_w1[prev_k]] + bias),  x_k = rms(h_k; norm)
//   prev_0 = anchor, prev_k = token k - 1 (the walk's);
//   length = first k with c_k < thr_k (thr_k > 0), else gamma.
// x_k is formed here from the final residual row h_k exactly (its own sum of
// squares), so the head reads the same final-normed rows as lm_head.
// One workgroup per draft row, wave w takes slots w, w + 16, ...; every lane
// holds H / 64 entries of the row.  grid A, block 1024
// ---------------------------------------------------------------------------
constexpr int CONF_NV = 4;  // 8-element pieces per lane and pass (H up to 64 * 8 * CONF_NV per pass)

__global__ __launch_bounds__(1024) void k_conf(const ConfArgs a) {
  __shared__ float cs[CONF_MAX_GAMMA];
  const int row = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, G = a.rows.gamma;
  if (a.head) {
    const float b = ld_act(a.bias, 0, a.act_bf16);
    const bool bf = a.act_bf16 != 0, wbf = a.wkind == WK_BF16;
    const int cols = a.H + (a.with_markov ? a.rank : 0);
    for (int k = wave; k < G; k += 16) {
      const int64_t m = (int64_t)row * G + k;
      const float* h = a.hn + m * a.ldh;
      float ss = 0.f, dot = 0.f;
      // pieces of eight: every load of a pass issued before the first use
      for (int p0 = 0; p0 < a.H; p0 += 64 * 8 * CONF_NV) {
        f32x4 hv[CONF_NV][2];
        Raw8 wn[CONF_NV];
        u32x4 pw[CONF_NV];
#pragma unroll
        for (int q = 0; q < CONF_NV; ++q) {
          const int i0 = min(p0 + 8 * (lane + 64 * q), a.H - 8);
          hv[q][0] = *(const f32x4*)(h + i0);
          hv[q][1] = *(const f32x4*)(h + i0 + 4);
          wn[q] = ld_act8(a.wnorm, i0, bf);
          if (wbf) pw[q] = *(const u32x4*)((const uint16_t*)a.pw + i0);
        }
#pragma unroll
        for (int q = 0; q < CONF_NV; ++q) {
          const int i0 = p0 + 8 * (lane + 64 * q);
          if (i0 >= a.H) break;
          float w8[8];
          cvt_act8(wn[q], bf, w8);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float v = hv[q][e >> 2][e & 3];
            const float p = wbf ? __uint_as_float((pw[q][e >> 1] << ((e & 1) ? 0 : 16)) & 0xFFFF0000u)
                                : table_elem(a.pw, a.ps, a.pb, a.wkind, a.group, 0, cols, i0 + e);
            ss += v * v;
            dot += v * w8[e] * p;
          }
        }
      }
      ss = wave_sum(ss);
      dot = wave_sum(dot) / sqrtf(ss / a.H + a.eps);
      if (a.with_markov) {
        const int prev = k == 0 ? a.rows.anchor[row] : a.tokens[m - 1];
        float dm = 0.f;
        if (prev >= 0)  // a walk step without a finite candidate reports -1 (no Markov feature)
          for (int j = lane; j < a.rank; j += 64)
            dm += table_elem(a.pw, a.ps, a.pb, a.wkind, a.group, 0, cols, a.H + j) *
                  table_elem(a.w1, a.w1s, a.w1b, a.wkind, a.group, prev, a.rank, j);
        dot += wave_sum(dm);
      }
      const float c = 1.f / (1.f + expf(-(dot + b)));
      if (lane == 0) {
        cs[k] = c;
        a.conf[m] = c;
      }
    }
  }
  __syncthreads();
  if (tid == 0 && a.lengths) {
    int len = G;
    if (a.head)
      for (int k = 0; k < G; ++k)
        if (a.thr[k] > 0.f && cs[k] < a.thr[k]) {
          len = k;
          break;
        }
    a.lengths[row] = len;
  }
}

// ---------------------------------------------------------------------------
hipError_t launch_conf(const ConfArgs& a, hipStream_t st) {
  if (a.rows.gamma > CONF_MAX_GAMMA || a.rows.A < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_conf, dim3(a.rows.A), dim3(1024), 0, st, a);
  return hipGetLastError();
}
hipError_t launch_embed(const EmbedArgs& a, int M, hipStream_t st) {
  hipLaunchKernelGGL(k_embed, dim3(M), dim3(256), 0, st, a);
  return hipGetLastError();
}
hipError_t launch_zero(unsigned* p, int64_t n, hipStream_t st) {
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(k_zero, dim3(blocks < 1 ? 1 : (blocks > 1024 ? 1024 : (unsigned)blocks)), dim3(256), 0, st, p, n);
  return hipGetLastError();
}
hipError_t launch_merge(const MergeArgs& a, hipStream_t st) {
  const int nrows = a.A * a.nKv * a.nq;
  if (nrows <= MERGE_FEW_ROWS) {
    // few rows: a workgroup per row keeps enough of the chip busy; rows
    // with more splits than one pass holds, in the wide attention's lane
    // order, go to k_merge_split (row-major partials: the short-context
    // kernel's at most 64 splits, where four thread groups gained nothing)
    int most = 0;
    for (int r = 0; r < a.A; ++r) most = std::max(most, a.split_off[r + 1] - a.split_off[r]);
    if (most > MERGE_RB && a.part_f16 && a.lane_order && a.hd % 32 == 0) {
      const int64_t units = (int64_t)a.A * a.nKv * ((a.nq + 15) / 16) * (a.hd / 32);
      hipLaunchKernelGGL((k_merge_split<16>), dim3((unsigned)units), dim3(1024), 0, st, a);
      return hipGetLastError();
    }
    if (a.part_f16 && a.lane_order) hipLaunchKernelGGL((k_merge_rows<true, true>), dim3(nrows), dim3(a.hd), 0, st, a);
    else if (a.part_f16) hipLaunchKernelGGL((k_merge_rows<true, false>), dim3(nrows), dim3(a.hd), 0, st, a);
    else hipLaunchKernelGGL((k_merge_rows<false, false>), dim3(nrows), dim3(a.hd), 0, st, a);
    return hipGetLastError();
  }
  const int per = 256 / (a.hd / 8);  // query rows per workgroup (row-major partials)
  if (a.part_f16 && a.lane_order) {
    const int64_t threads = (int64_t)a.A * a.nKv * ((a.nq + 15) / 16) * (a.hd / 32) * 64;
    hipLaunchKernelGGL((k_merge<true, true>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, a);
  } else if (a.part_f16) {
    hipLaunchKernelGGL((k_merge<true, false>), dim3((nrows + per - 1) / per), dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL((k_merge<false, false>), dim3((nrows + per - 1) / per), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}
hipError_t launch_walk(const WalkArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_walk, dim3(a.rows.A), dim3(WALK_NT), 0, st, a);
  return hipGetLastError();
}
hipError_t launch_aux(const AuxArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_aux, dim3((a.V + 3) / 4), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace dsp
