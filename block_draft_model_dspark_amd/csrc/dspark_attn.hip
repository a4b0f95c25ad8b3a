// ctx++block attention of the draft round on bf16 MFMA.
//
// deepspec-module.ts, plainDeepspecContext.attend / deepspec.ts,
// #forwardBackbone: for draft row a, O = softmax(q K^T) V with scale 1.0, no
// mask, over [row a's context K/V ++ its own gamma block keys]; all query
// heads of a KV group read that group's single K/V head.
//
// Layout: one workgroup per (row, key split, kv head); wave w owns 16 query
// rows of the group (row index hl*gamma + g).  Keys stream through LDS in
// chunks: K rows as is, V transposed (Vt[d][key]).  Scores are computed as
// S^T = K q^T so that each lane holds one query column and the softmax max
// is a 2-step lane exchange; the output is O^T = V^T P^T.  Query rows and
// probabilities are fp32 split into bf16 hi + lo (two MFMAs); the bf16
// context cache is exact in one plane.  fp32 keys (the block's own keys, or
// an fp32 cache) go in 16-key chunks as hi and lo planes: the score adds
// K_lo q_hi, and V hi/lo planes sit in the two k-halves of one MFMA against
// duplicated probabilities, so one MFMA sums both.
// Each workgroup writes unnormalised O with its (max, sum); k_merge combines
// the splits.
#include "dspark_kernels.hpp"
#include "dspark_common.hpp"

namespace dsp {

template <int HD, bool KVB>
__global__ __launch_bounds__(512) void k_attn(const AttnArgs a) {
  constexpr int NS = HD / 32;   // 32-wide hd steps of the score MFMAs
  constexpr int NT = HD / 16;   // 16-row hd tiles of the output
  constexpr int KSTR = HD + 8;  // Ks row stride (bf16)
  constexpr int VSTR = 40;      // Vt row stride (bf16): 32 keys + pad
  __shared__ __align__(16) uint16_t Ks[32 * KSTR];
  __shared__ __align__(16) uint16_t Vt[HD * VSTR];

  const int sg = blockIdx.x, kvh = blockIdx.y;
  int row = 0;
  while (a.split_off[row + 1] <= sg) ++row;
  const int sp = sg - a.split_off[row];
  const int len = a.len[row];
  const int T = len + a.gamma;
  const int j0 = sp * a.split, j1 = min(T, j0 + a.split);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, gq = lane >> 4, ln = lane & 15;
  const int qrow = wave * 16 + ln;
  const bool qok = qrow < a.nq;

  // query operand (B of S^T = K q^T): col = query row, k = hd 32s + 8gq..
  bf16x8 qh[NS], ql[NS];
  {
    const float* qp = a.q + (((int64_t)row * a.nKv + kvh) * a.nq + (qok ? qrow : 0)) * HD;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      float t[8];
      if (qok) {
        f32x4 x0 = *(const f32x4*)(qp + 32 * s + 8 * gq), x1 = *(const f32x4*)(qp + 32 * s + 8 * gq + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) { t[e] = x0[e]; t[4 + e] = x1[e]; }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) t[e] = 0.f;
      }
      split8(t, qh[s], ql[s]);
    }
  }

  f32x4 o[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_part = 0.f;

  const int64_t kvoff = (int64_t)kvh * len * HD;
  const uint16_t* kc16 = (const uint16_t*)a.row[row].k + kvoff;
  const uint16_t* vc16 = (const uint16_t*)a.row[row].v + kvoff;
  const float* kc32 = (const float*)a.row[row].k + kvoff;
  const float* vc32 = (const float*)a.row[row].v + kvoff;
  const float* kbp = a.kb + ((int64_t)row * a.nKv + kvh) * a.gamma * HD;
  const float* vbp = a.vb + ((int64_t)row * a.nKv + kvh) * a.gamma * HD;
  const int nthr = blockDim.x;

  for (int jc = j0; jc < j1;) {
    const bool one = KVB && jc < len;  // bf16 context keys: one plane, 32 keys
    const int jend = one ? min(min(j1, len), jc + 32) : min(j1, jc + 16);
    const int nvalid = jend - jc;

    __syncthreads();
    if (one) {
      for (int u = tid; u < 32 * (HD / 8); u += nthr) {
        const int r = u / (HD / 8), c8 = u - r * (HD / 8);
        u32x4 kk = u32x4{0u, 0u, 0u, 0u}, vv = u32x4{0u, 0u, 0u, 0u};
        if (r < nvalid) {
          kk = *(const u32x4*)(kc16 + (int64_t)(jc + r) * HD + 8 * c8);
          vv = *(const u32x4*)(vc16 + (int64_t)(jc + r) * HD + 8 * c8);
        }
        *(u32x4*)&Ks[r * KSTR + 8 * c8] = kk;
#pragma unroll
        for (int e = 0; e < 8; ++e) Vt[(8 * c8 + e) * VSTR + r] = (uint16_t)(vv[e >> 1] >> (16 * (e & 1)));
      }
    } else {
      for (int u = tid; u < 16 * (HD / 8); u += nthr) {
        const int r = u / (HD / 8), c8 = u - r * (HD / 8);
        float kf[8], vf[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) { kf[e] = 0.f; vf[e] = 0.f; }
        if (r < nvalid) {
          const int j = jc + r;
          const float* ks = j < len ? kc32 + (int64_t)j * HD : kbp + (int64_t)(j - len) * HD;
          const float* vs = j < len ? vc32 + (int64_t)j * HD : vbp + (int64_t)(j - len) * HD;
          f32x4 k0 = *(const f32x4*)(ks + 8 * c8), k1 = *(const f32x4*)(ks + 8 * c8 + 4);
          f32x4 v0 = *(const f32x4*)(vs + 8 * c8), v1 = *(const f32x4*)(vs + 8 * c8 + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) { kf[e] = k0[e]; kf[4 + e] = k1[e]; vf[e] = v0[e]; vf[4 + e] = v1[e]; }
        }
        bf16x8 kh, kl, vh, vl;
        split8(kf, kh, kl);
        split8(vf, vh, vl);
        *(u32x4*)&Ks[r * KSTR + 8 * c8] = __builtin_bit_cast(u32x4, kh);
        *(u32x4*)&Ks[(16 + r) * KSTR + 8 * c8] = __builtin_bit_cast(u32x4, kl);
        // halves are taken from the whole-vector bit pattern (bit-casting a
        // single __bf16 vector element is lowered to element 0 by this compiler)
        const u32x4 vhw = __builtin_bit_cast(u32x4, vh), vlw = __builtin_bit_cast(u32x4, vl);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          Vt[(8 * c8 + e) * VSTR + r] = (uint16_t)(vhw[e >> 1] >> (16 * (e & 1)));
          Vt[(8 * c8 + e) * VSTR + 16 + r] = (uint16_t)(vlw[e >> 1] >> (16 * (e & 1)));
        }
      }
    }
    __syncthreads();

    // scores S^T (rows = keys, cols = queries)
    float sv[8];
    {
      f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const bf16x8 k0 = __builtin_bit_cast(bf16x8, *(const u32x4*)&Ks[ln * KSTR + 32 * s + 8 * gq]);
        const bf16x8 k1 = __builtin_bit_cast(bf16x8, *(const u32x4*)&Ks[(16 + ln) * KSTR + 32 * s + 8 * gq]);
        s0 = mfma16(k0, qh[s], s0);
        s0 = mfma16(k0, ql[s], s0);
        if (one) {
          s1 = mfma16(k1, qh[s], s1);
          s1 = mfma16(k1, ql[s], s1);
        } else {
          s0 = mfma16(k1, qh[s], s0);  // K_lo q_hi
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[i] = (4 * gq + i < nvalid) ? s0[i] : -INFINITY;
        sv[4 + i] = (one && 16 + 4 * gq + i < nvalid) ? s1[i] : -INFINITY;
      }
    }

    // online softmax for this lane's query column
    float mx = sv[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sv[e]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(m_run, mx);
    if (mnew > m_run) {
      const float sc = expf(m_run - mnew);
#pragma unroll
      for (int t = 0; t < NT; ++t) o[t] *= sc;
      l_part *= sc;
      m_run = mnew;
    }
    float pe[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = expf(sv[e] - m_run);
      l_part += p;
      pe[e] = p;
    }
    if (!one) {
#pragma unroll
      for (int e = 0; e < 4; ++e) pe[4 + e] = pe[e];
    }
    bf16x8 ph, pl;
    split8(pe, ph, pl);

    // O^T += V^T P^T
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int hr = 16 * t + ln;
      const u32x2 va = *(const u32x2*)&Vt[hr * VSTR + 4 * gq];
      const u32x2 vb = *(const u32x2*)&Vt[hr * VSTR + 16 + 4 * gq];
      const bf16x8 vop = __builtin_bit_cast(bf16x8, u32x4{va[0], va[1], vb[0], vb[1]});
      o[t] = mfma16(vop, ph, o[t]);
      o[t] = mfma16(vop, pl, o[t]);
    }
    jc = jend;
  }

  float l = l_part;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (qok) {
    const int64_t base = ((int64_t)sg * a.nKv + kvh) * a.nq + qrow;
#pragma unroll
    for (int t = 0; t < NT; ++t) *(f32x4*)&a.opart[base * HD + 16 * t + 4 * gq] = o[t];
    if (gq == 0) {
      a.ml[base * 2] = m_run;
      a.ml[base * 2 + 1] = l;
    }
  }
}

hipError_t launch_attn(const AttnArgs& a, int hd, bool kv_bf16, int nsplit, hipStream_t st) {
  const int waves = (a.nq + 15) / 16;
  dim3 grid(nsplit, a.nKv), block(64 * waves);
#define DSP_ATTN(H)                                                                            \
  if (kv_bf16) hipLaunchKernelGGL((k_attn<H, true>), grid, block, 0, st, a);                   \
  else hipLaunchKernelGGL((k_attn<H, false>), grid, block, 0, st, a);
  if (hd == 64) { DSP_ATTN(64) }
  else if (hd == 128) { DSP_ATTN(128) }
  else { DSP_ATTN(256) }
#undef DSP_ATTN
  return hipGetLastError();
}

}  // namespace dsp
