// ctx++block attention of the draft round on bf16 MFMA.
//
// deepspec-module.ts, plainDeepspecContext.attend / deepspec.ts,
// #forwardBackbone: for draft row a, O = softmax(q K^T) V with scale 1.0, no
// mask, over [row a's context K/V ++ its own gamma block keys]; all query
// heads of a KV group read that group's single K/V head.
//
// Layout: one workgroup per (row, key split, kv head, 16 query rows) (query
// row index hl*gamma + g).  A row's context keys are cut into splits of
// a.split keys and its block keys form one more split.  The workgroup loads
// its 16 query rows once (RMS factor applied, split into bf16 hi + lo) into
// LDS; keys go through LDS in chunks of 32, all loads of a chunk issued
// before the first LDS write: K rows as is, V transposed (Vt[d][key]).  Every
// wave forms the scores S^T = K q^T of the chunk (each lane holds one query
// column; the softmax max is a 2-step lane exchange) and the output for its
// quarter of the head dimension, O^T = V^T P^T.  Probabilities are fp32
// split into hi + lo (two MFMAs); the bf16 context cache is exact in one
// plane.  fp32 keys (the block's own keys, or an fp32 cache) go in 16-key
// passes as hi and lo planes: the score adds K_lo q_hi, and V hi/lo planes
// sit in the two k-halves of one MFMA against duplicated probabilities, so
// one MFMA sums both.
//
// The q|k GEMM leaves q and the block's k, v without their per-head RMS
// factor (a per-row scalar); it is formed here from the stored sums of
// squares and applied as q and the block keys are loaded.
// Each workgroup writes unnormalised O with its (max, sum); k_merge combines
// the splits.
#include "dspark_kernels.hpp"
#include "dspark_common.hpp"

namespace dsp {

constexpr int ATT_NTH = 256;  // threads per workgroup (4 waves, one quarter of hd each)
constexpr float ATT_LOG2E = 1.4426950408889634f;
constexpr float ATT_RESCALE = 8.f;  // slack of the softmax reference max (natural-log units)

// one pass over the keys staged in LDS: ONE = 32 one-plane keys, else 16
// keys as hi (rows 0..15) and lo (rows 16..31) planes.  o: this wave's NTW
// output tiles (head dims 16 t0 + 16 t ..).
template <int HD, bool ONE, int NTW>
__device__ __forceinline__ void attn_pass(const uint16_t* Ks, const uint16_t* Vt, const bf16x8* qh, const bf16x8* ql,
                                          f32x4* o, int t0, float& m_run, float& l_part, int nvalid) {
  constexpr int NS = HD / 32, KSTR = HD + 8, VSTR = 40;
  const int lane = threadIdx.x & 63, gq = lane >> 4, ln = lane & 15;
  float sv[8];
  {
    f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const bf16x8 k0 = __builtin_bit_cast(bf16x8, *(const u32x4*)&Ks[ln * KSTR + 32 * s + 8 * gq]);
      const bf16x8 k1 = __builtin_bit_cast(bf16x8, *(const u32x4*)&Ks[(16 + ln) * KSTR + 32 * s + 8 * gq]);
      s0 = mfma16(k0, qh[s], s0);
      s0 = mfma16(k0, ql[s], s0);
      if constexpr (ONE) {
        s1 = mfma16(k1, qh[s], s1);
        s1 = mfma16(k1, ql[s], s1);
      } else {
        s0 = mfma16(k1, qh[s], s0);  // K_lo q_hi
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = (4 * gq + i < nvalid) ? s0[i] : -INFINITY;
      sv[4 + i] = (ONE && 16 + 4 * gq + i < nvalid) ? s1[i] : -INFINITY;
    }
  }
  // online softmax for this lane's query column.  The reference max m_run
  // moves only when a chunk's max passes it by more than ATT_RESCALE, so the
  // O rescale (a multiply per accumulator) runs after the first chunk only
  // rarely; probabilities stay below e^ATT_RESCALE, and (m_run, l) stay
  // consistent for the merge whatever reference was used.  exp(x) is the
  // hardware 2^(x log2 e).
  float mx = sv[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sv[e]);
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  if (mx > m_run + ATT_RESCALE) {
    const float sc = __builtin_amdgcn_exp2f((m_run - mx) * ATT_LOG2E);
#pragma unroll
    for (int t = 0; t < NTW; ++t) o[t] *= sc;
    l_part *= sc;
    m_run = mx;
  }
  const float mb = m_run * ATT_LOG2E;
  float pe[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float p = __builtin_amdgcn_exp2f(fmaf(sv[e], ATT_LOG2E, -mb));
    l_part += p;
    pe[e] = p;
  }
  if constexpr (!ONE) {
#pragma unroll
    for (int e = 0; e < 4; ++e) pe[4 + e] = pe[e];
  }
  bf16x8 ph, pl;
  split8(pe, ph, pl);
  // O^T += V^T P^T over this wave's head dims
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const int hr = 16 * (t0 + t) + ln;
    bf16x8 vop;
    if constexpr (ONE) {
      // one-plane chunks store V^T with keys in the score layout's k-slot
      // order (slot 8g + e: key 4g + e, then 16 + 4g + e - 4), one 16-byte read
      vop = __builtin_bit_cast(bf16x8, *(const u32x4*)&Vt[hr * VSTR + 8 * gq]);
    } else {
      const u32x2 va = *(const u32x2*)&Vt[hr * VSTR + 4 * gq];
      const u32x2 vb = *(const u32x2*)&Vt[hr * VSTR + 16 + 4 * gq];
      vop = __builtin_bit_cast(bf16x8, u32x4{va[0], va[1], vb[0], vb[1]});
    }
    o[t] = mfma16(vop, ph, o[t]);
    o[t] = mfma16(vop, pl, o[t]);
  }
}

__device__ __forceinline__ uint16_t half_of(const u32x4& w, int e) { return (uint16_t)(w[e >> 1] >> (16 * (e & 1))); }

// The keys of one split: every load of chunk c + 1 is issued before chunk c's
// MFMAs, and chunk 0's before the query operand is formed (prep fills qh,
// ql; a wave's loads complete in order, so the query loads went first).
// ONE: bf16 context keys, 32 per pass in one plane; else fp32 keys (the
// block's own, scaled by their RMS factor: rkey for this thread's key, or an
// fp32 cache: 1) in two 16-key passes of hi / lo planes.  NTH threads stage;
// each wave accumulates NTW output tiles from t0.
// V-only cache (VO): the keys are rebuilt while staging as
// K = RoPE(V * k_norm, pos0 + j) (deepspec.ts, #projectContextKVRows: V is
// the weightless norm of the same k whose k_norm'd, roped form is K).  Thread
// items c8 = tid / 32 + (NTH / 32) i hold dims 8 c8..; items i and i + PI are
// the two halves of the same RoPE pairs when (HD / 16) is a multiple of
// NTH / 32 (vo_layout_ok), so each thread rotates its own values.
template <int HD, int NTH>
__host__ __device__ constexpr bool vo_layout_ok() {
  return (HD / 16) % (NTH / ATT_KEYS) == 0 && ATT_KEYS * (HD / 8) % NTH == 0;
}
struct VoCtx {
  const uint32_t* knw;  // LDS: k_norm as bf16 pairs [HD / 2]
  const double* inv;    // LDS: 1 / wavelength per pair [HD / 2] (0: identity)
  int64_t pos0;         // absolute position of context key 0 of the row
};

template <int HD, bool ONE, int NTH, int NTW, bool VO = false, class Prep>
__device__ __forceinline__ void attn_keys(const void* kbase, const void* vbase, int j0, int j1, float rkey,
                                          Prep&& prep, const bf16x8* qh, const bf16x8* ql, f32x4* o, int t0,
                                          float& m_run, float& l_part, uint16_t* Ks, uint16_t* Vt,
                                          const VoCtx& vo = VoCtx{}) {
  constexpr int KSTR = HD + 8, VSTR = 40;
  constexpr int IPT = ATT_KEYS * (HD / 8) / NTH;  // staging items (key, 8 dims) per thread
  static_assert(IPT >= 1 && ATT_KEYS * (HD / 8) % NTH == 0 && NTH % ATT_KEYS == 0, "staging layout");
  static_assert(!VO || (ONE && vo_layout_ok<HD, NTH>()), "V-only staging: bf16 cache, pairs within a thread");
  const int tid = threadIdx.x;
  const int key = tid & (ATT_KEYS - 1);  // the key this thread stages (all its items)
  u32x4 kk[ONE ? IPT : 1], vv[ONE ? IPT : 1];
  f32x4 kf[ONE ? 1 : IPT][2], vf[ONE ? 1 : IPT][2];
  auto load = [&](int jc) {
    const int kc = jc + min(key, j1 - jc - 1);
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      const int c8 = (tid + NTH * i) / ATT_KEYS;
      if constexpr (ONE) {
        if constexpr (!VO) kk[i] = *(const u32x4*)((const uint16_t*)kbase + (int64_t)kc * HD + 8 * c8);
        vv[i] = *(const u32x4*)((const uint16_t*)vbase + (int64_t)kc * HD + 8 * c8);
      } else {
        const float* kp = (const float*)kbase + (int64_t)kc * HD + 8 * c8;
        const float* vp = (const float*)vbase + (int64_t)kc * HD + 8 * c8;
        kf[i][0] = *(const f32x4*)kp;
        kf[i][1] = *(const f32x4*)(kp + 4);
        vf[i][0] = *(const f32x4*)vp;
        vf[i][1] = *(const f32x4*)(vp + 4);
      }
    }
  };
  load(j0);
  prep();
  for (int jc = j0; jc < j1; jc += ATT_KEYS) {
    const int nk = min(ATT_KEYS, j1 - jc);
    const bool ok = key < nk;
    if constexpr (ONE) {
      if constexpr (VO) {
        // K of this thread's key from its V: items i < PI hold dims
        // [0, HD/2) of the pairs, items i + PI the partner dims
        constexpr int PI = (HD / 16) / (NTH / ATT_KEYS);
        const int64_t pos = vo.pos0 + jc + min(key, j1 - jc - 1);
#pragma unroll
        for (int i = 0; i < PI; ++i) {
          const int c8 = (tid + NTH * i) / ATT_KEYS;  // dims 8 c8 .. in the first half
          const u32x4 wl = *(const u32x4*)&vo.knw[4 * c8], wh = *(const u32x4*)&vo.knw[HD / 4 + 4 * c8];
          float klo[8], khi[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t sh = (e & 1) ? 0u : 16u;  // bf16 e of a word: low half first
            const float vlo = __uint_as_float((vv[i][e >> 1] << sh) & 0xFFFF0000u);
            const float vhi = __uint_as_float((vv[i + PI][e >> 1] << sh) & 0xFFFF0000u);
            const float tl = vlo * __uint_as_float((wl[e >> 1] << sh) & 0xFFFF0000u);
            const float th = vhi * __uint_as_float((wh[e >> 1] << sh) & 0xFFFF0000u);
            float c, sn;
            rope_cs_hw(pos, vo.inv[8 * c8 + e], c, sn);
            klo[e] = tl * c - th * sn;
            khi[e] = th * c + tl * sn;
          }
          kk[i] = __builtin_bit_cast(u32x4, to_bf16x8(klo));
          kk[i + PI] = __builtin_bit_cast(u32x4, to_bf16x8(khi));
        }
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < IPT; ++i) {
        // keys past the chunk hold a copy of its last key: their scores are
        // masked to -inf, so their probabilities are exactly 0
        const int c8 = (tid + NTH * i) / ATT_KEYS;
        *(u32x4*)&Ks[key * KSTR + 8 * c8] = kk[i];
        const u32x4 vw = vv[i];
        // V^T in 32-bit words of two keys: the lanes of keys 2k and 2k + 1
        // (adjacent lanes, same dims) swap half their dims, then the even
        // lane writes dims 0..3 and the odd lane dims 4..7 of the pair
        const bool odd = key & 1;
        const uint32_t s0 = odd ? vw[0] : vw[2], s1 = odd ? vw[1] : vw[3];
        const uint32_t r0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)s0, 0xB1, 0xF, 0xF, false);  // lane ^ 1
        const uint32_t r1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)s1, 0xB1, 0xF, 0xF, false);
        const uint32_t m0 = odd ? vw[2] : vw[0], m1 = odd ? vw[3] : vw[1];  // this lane's four dims
        const int e0 = odd ? 4 : 0;
        // k-slot of the pair's even key: keys 4g.. of each half of the chunk
        // take slots 8g.. (first half) and 8g + 4.. (second half)
        const int k2 = key & ~1, slot = 8 * ((k2 & 15) >> 2) + 4 * (k2 >> 4) + (k2 & 3);
        uint32_t* vrow = (uint32_t*)&Vt[(8 * c8 + e0) * VSTR + slot];
        const uint32_t mine[4] = {m0 & 0xFFFFu, m0 >> 16, m1 & 0xFFFFu, m1 >> 16};
        const uint32_t part[4] = {r0 & 0xFFFFu, r0 >> 16, r1 & 0xFFFFu, r1 >> 16};
#pragma unroll
        for (int e = 0; e < 4; ++e) vrow[e * (VSTR / 2)] = odd ? (part[e] | (mine[e] << 16)) : (mine[e] | (part[e] << 16));
      }
      __syncthreads();
      if (jc + ATT_KEYS < j1) load(jc + ATT_KEYS);
      attn_pass<HD, true, NTW>(Ks, Vt, qh, ql, o, t0, m_run, l_part, nk);
    } else {
      float kv8[IPT][8], vv8[IPT][8];
      const float sc = ok ? rkey : 0.f;
#pragma unroll
      for (int i = 0; i < IPT; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kv8[i][e] = kf[i][0][e] * sc;
          kv8[i][4 + e] = kf[i][1][e] * sc;
          vv8[i][e] = vf[i][0][e] * sc;
          vv8[i][4 + e] = vf[i][1][e] * sc;
        }
      if (jc + ATT_KEYS < j1) load(jc + ATT_KEYS);
      for (int pass = 0; pass < 2 && 16 * pass < nk; ++pass) {
        __syncthreads();
        if ((key >> 4) == pass) {
          const int rr = key & 15;
#pragma unroll
          for (int i = 0; i < IPT; ++i) {
            const int c8 = (tid + NTH * i) / ATT_KEYS;
            bf16x8 kh, kl, vh, vl;
            split8(kv8[i], kh, kl);
            split8(vv8[i], vh, vl);
            *(u32x4*)&Ks[rr * KSTR + 8 * c8] = __builtin_bit_cast(u32x4, kh);
            *(u32x4*)&Ks[(16 + rr) * KSTR + 8 * c8] = __builtin_bit_cast(u32x4, kl);
            // halves are taken from the whole-vector bit pattern (bit-casting a
            // single __bf16 vector element is lowered to element 0 by this compiler)
            const u32x4 vhw = __builtin_bit_cast(u32x4, vh), vlw = __builtin_bit_cast(u32x4, vl);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              Vt[(8 * c8 + e) * VSTR + rr] = half_of(vhw, e);
              Vt[(8 * c8 + e) * VSTR + 16 + rr] = half_of(vlw, e);
            }
          }
        }
        __syncthreads();
        attn_pass<HD, false, NTW>(Ks, Vt, qh, ql, o, t0, m_run, l_part, min(16, nk - 16 * pass));
      }
    }
  }
}

// This lane's output tiles t0.. (dims 16 t + 4 (lane / 16) .. + 3 of its
// query).  An fp32 cache stores the fp32 sums at [split, kvh, nq, hd] (element
// offset off32 of this lane's first dim).  A bf16 cache stores fp16 O / l
// (bounded by the largest |v|, so in range; half the bytes): LANE = false at
// [split, kvh, nq, hd] like the fp32 sums; LANE = true in the lanes' own
// order, [split, kvh, query group of 16, tile pair, lane, 8] with tile 2j in
// halves 0..3 and tile 2j + 1 in halves 4..7 (element offset offp of this
// (split, kvh, group), pair 0, lane 0), so a wave's store of a tile pair is
// 1 KiB contiguous (the merge then reads 16-byte pieces of several rows).
template <bool F16, bool LANE, int HD, int NTW>
__device__ __forceinline__ void store_part(void* opart, int64_t off32, int64_t offp, int t0, const f32x4 (&o)[NTW],
                                           float l) {
  if constexpr (F16 && !LANE) {
    const float rl = 1.f / l;
#pragma unroll
    for (int t = 0; t < NTW; ++t)
      *(u32x2*)((uint16_t*)opart + off32 + 16 * (t0 + t)) =
          u32x2{pack_f16x2(o[t][0] * rl, o[t][1] * rl), pack_f16x2(o[t][2] * rl, o[t][3] * rl)};
  } else if constexpr (F16) {
    const float rl = 1.f / l;
    const int lane = threadIdx.x & 63;
    uint16_t* const base = (uint16_t*)opart + offp + 8 * lane;
    if constexpr (NTW % 2 == 0) {  // t0 even: whole pairs
#pragma unroll
      for (int t = 0; t < NTW; t += 2)
        *(u32x4*)(base + (int64_t)((t0 + t) / 2) * 512) =
            u32x4{pack_f16x2(o[t][0] * rl, o[t][1] * rl), pack_f16x2(o[t][2] * rl, o[t][3] * rl),
                  pack_f16x2(o[t + 1][0] * rl, o[t + 1][1] * rl), pack_f16x2(o[t + 1][2] * rl, o[t + 1][3] * rl)};
    } else {
#pragma unroll
      for (int t = 0; t < NTW; ++t)
        *(u32x2*)(base + (int64_t)((t0 + t) / 2) * 512 + 4 * ((t0 + t) & 1)) =
            u32x2{pack_f16x2(o[t][0] * rl, o[t][1] * rl), pack_f16x2(o[t][2] * rl, o[t][3] * rl)};
    }
  } else {
#pragma unroll
    for (int t = 0; t < NTW; ++t) *(f32x4*)((float*)opart + off32 + 16 * (t0 + t)) = o[t];
  }
}

// V-only cache: the workgroup's RoPE inverse wavelengths and k_norm weight
// in LDS (filled before the first barrier of the key loop)
template <int HD, bool VO>
struct VoTables {
  __align__(16) uint32_t knw[VO ? HD / 2 : 1];
  double inv[VO ? HD / 2 : 1];
};
template <int HD, bool VO>
__device__ __forceinline__ VoCtx vo_setup(VoTables<HD, VO>& t, const AttnArgs& a, int row) {
  VoCtx v{};
  if constexpr (VO) {
    const int tid = threadIdx.x;
    if (tid < HD / 2) {
      t.knw[tid] = ((const uint32_t*)a.kn)[tid];
      t.inv[tid] = rope_inv(tid, a.rope_step, a.nrot);
    }
    __syncthreads();  // (called by every thread of the workgroup: the split kind is uniform)
    v.knw = t.knw;
    v.inv = t.inv;
    v.pos0 = a.ctx_pos0[row];
  }
  return v;
}

template <int HD, bool KVB, bool VO>
__global__ __launch_bounds__(ATT_NTH) void k_attn(const AttnArgs a) {
  constexpr int NS = HD / 32, NTW = HD / 64, HJ = HD / 64;
  static_assert(ATT_KEYS * (HD / 8) / ATT_NTH >= 1 && ATT_NTH % ATT_KEYS == 0, "staging layout");
  __shared__ __align__(16) uint16_t Ks[32 * (HD + 8)];
  __shared__ __align__(16) uint16_t Vt[HD * 40];
  __shared__ __align__(16) u32x4 qop[2][NS][64];  // q hi / lo in B-operand order
  __shared__ VoTables<HD, VO> vot;

  const int sg = blockIdx.x, kvh = blockIdx.y;
  int row = 0;
  while (a.split_off[row + 1] <= sg) ++row;
  const int sp = sg - a.split_off[row];
  const bool blk = sp == a.split_off[row + 1] - a.split_off[row] - 1;  // the row's block keys
  const int len = a.len[row];
  const int j0 = blk ? 0 : sp * a.split, j1 = blk ? a.gamma : min(len, j0 + a.split);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, gq = lane >> 4, ln = lane & 15;
  const int rep = a.nH / a.nKv;
  const int q0 = blockIdx.z * 16;  // first query row of the workgroup

  // 1. the workgroup's 16 query rows, as items (query, 8 dims): their loads
  //    and the rows' sums of squares first, then the first keys' loads
  constexpr int QC8 = HD / 8, QIT = (16 * QC8 + ATT_NTH - 1) / ATT_NTH;  // items per thread
  f32x4 qv[QIT][2];
  float qss[QIT];
#pragma unroll
  for (int k = 0; k < QIT; ++k) {
    const int it = min(tid + ATT_NTH * k, 16 * QC8 - 1);
    const int qi = it / QC8, c8 = it - qi * QC8;
    const int qr = min(q0 + qi, a.nq - 1);
    const int hl = qr / a.gamma, g = qr - hl * a.gamma, head = kvh * rep + hl;
    const float* qp = a.q + (((int64_t)row * a.nKv + kvh) * a.nq + qr) * HD + 8 * c8;
    qv[k][0] = *(const f32x4*)qp;
    qv[k][1] = *(const f32x4*)(qp + 4);
    float ss = 0.f;
#pragma unroll
    for (int p = 0; p < HJ; ++p) ss += a.ssq[(int64_t)(head * HJ + p) * a.M + row * a.gamma + g];
    qss[k] = ss;
  }
  // RMS factor of the block key this thread stages (k_norm / weightless v
  // share it)
  const int key = tid & (ATT_KEYS - 1);
  float sk = 0.f;
  if (blk) {
    const int kq = min(key, a.gamma - 1);
#pragma unroll
    for (int p = 0; p < HJ; ++p) sk += a.ssq[(int64_t)((a.nH + kvh) * HJ + p) * a.M + row * a.gamma + kq];
  }
  // q hi / lo into LDS: element (query qi, dim d) is B-operand lane
  // qi + 16 ((d mod 32) / 8), word d mod 8, of k-step d / 32; then every
  // wave takes the whole operand
  bf16x8 qh[NS], ql[NS];
  auto prep = [&]() {
#pragma unroll
    for (int k = 0; k < QIT; ++k) {
      const int it = tid + ATT_NTH * k;
      if (it < 16 * QC8) {
        const int qi = it / QC8, c8 = it - qi * QC8, d = 8 * c8;
        const float r = q0 + qi < a.nq ? 1.f / sqrtf(qss[k] / HD + a.eps) : 0.f;
        float t[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          t[e] = qv[k][0][e] * r;
          t[4 + e] = qv[k][1][e] * r;
        }
        bf16x8 h, l;
        split8(t, h, l);
        qop[0][d >> 5][qi + 16 * ((d & 31) >> 3)] = __builtin_bit_cast(u32x4, h);
        qop[1][d >> 5][qi + 16 * ((d & 31) >> 3)] = __builtin_bit_cast(u32x4, l);
      }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      qh[s] = __builtin_bit_cast(bf16x8, qop[0][s][lane]);
      ql[s] = __builtin_bit_cast(bf16x8, qop[1][s][lane]);
    }
  };

  f32x4 o[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_part = 0.f;
  const int t0 = wave * NTW;  // this wave's first 16-dim output tile

  if (blk) {
    const int64_t off = ((int64_t)row * a.nKv + kvh) * a.gamma * HD;
    attn_keys<HD, false, ATT_NTH, NTW>(a.kb + off, a.vb + off, j0, j1, 1.f / sqrtf(sk / HD + a.eps), prep, qh, ql,
                                       o, t0, m_run, l_part, Ks, Vt);
  } else {
    const int64_t kvoff = (int64_t)kvh * len * HD * (KVB ? 2 : 4);
    const char* vb = (const char*)a.row[row].v + kvoff;
    if constexpr (VO) {
      const VoCtx vo = vo_setup<HD, VO>(vot, a, row);
      attn_keys<HD, KVB, ATT_NTH, NTW, true>(vb, vb, j0, j1, 1.f, prep, qh, ql, o, t0, m_run, l_part, Ks, Vt, vo);
    } else {
      const char* kb = (const char*)a.row[row].k + kvoff;
      attn_keys<HD, KVB, ATT_NTH, NTW>(kb, vb, j0, j1, 1.f, prep, qh, ql, o, t0, m_run, l_part, Ks, Vt);
    }
  }

  float l = l_part;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  const int qrow = q0 + ln;
  if (qrow < a.nq) {
    const int64_t base = ((int64_t)sg * a.nKv + kvh) * a.nq + qrow;
    const int64_t grp = ((int64_t)sg * a.nKv + kvh) * ((a.nq + 15) / 16) + blockIdx.z;
    store_part<KVB, false, HD>(a.opart, base * HD + 4 * gq, grp * 16 * HD, t0, o, l);
    if (wave == 0 && gq == 0) {
      a.ml[base * 2] = m_run;
      a.ml[base * 2 + 1] = l;
    }
  }
}

// Many keys per row (a batch of long contexts): one workgroup per (row, key
// split, kv head) holding every query row of the group, wave w the 16 rows
// 16w.. over the whole head dimension.  Each staged key chunk then serves all
// query rows, and no wave repeats another's scores.  The query operand is
// loaded straight into B-operand order (lane: query l mod 16, dims
// 32s + 8(l / 16) ..), scaled by its RMS factor and split into hi / lo.
template <int HD, bool KVB, int NQT, bool VO>
__global__ __launch_bounds__(64 * NQT) void k_attn_wide(const AttnArgs a) {
  constexpr int NTH = 64 * NQT, NS = HD / 32, NTW = HD / 16, HJ = HD / 64;
  __shared__ __align__(16) uint16_t Ks[32 * (HD + 8)];
  __shared__ __align__(16) uint16_t Vt[HD * 40];
  __shared__ VoTables<HD, VO> vot;

  const int kvh = blockIdx.y;
  int sg = blockIdx.x, row = 0;
  if (a.xcd_rows) {
    // slot x / 8 among the splits of rows x mod 8, x mod 8 + 8, ...
    int slot = (int)(blockIdx.x >> 3);
    sg = -1;
    for (int r = blockIdx.x & 7; r < a.A; r += 8) {
      const int n = a.split_off[r + 1] - a.split_off[r];
      if (slot < n) {
        sg = a.split_off[r] + slot;
        row = r;
        break;
      }
      slot -= n;
    }
    if (sg < 0) return;  // an idle slot of a less loaded XCD (uniform: no barrier reached)
  } else {
    while (a.split_off[row + 1] <= sg) ++row;
  }
  const int sp = sg - a.split_off[row];
  const bool blk = sp == a.split_off[row + 1] - a.split_off[row] - 1;  // the row's block keys
  const int len = a.len[row];
  const int j0 = blk ? 0 : sp * a.split, j1 = blk ? a.gamma : min(len, j0 + a.split);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, gq = lane >> 4, ln = lane & 15;
  const int rep = a.nH / a.nKv;
  const int qr = wave * 16 + ln;  // this lane's query row (nq == 16 NQT)
  const int hl = qr / a.gamma, g = qr - hl * a.gamma, head = kvh * rep + hl;

  // 1. this lane's query dims and the row's sums of squares, then (inside
  //    attn_keys) the first keys' loads, then the operand is formed
  const float* qp = a.q + (((int64_t)row * a.nKv + kvh) * a.nq + qr) * HD + 8 * gq;
  f32x4 qv[NS][2];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    qv[s][0] = *(const f32x4*)(qp + 32 * s);
    qv[s][1] = *(const f32x4*)(qp + 32 * s + 4);
  }
  float qss = 0.f;
#pragma unroll
  for (int p = 0; p < HJ; ++p) qss += a.ssq[(int64_t)(head * HJ + p) * a.M + row * a.gamma + g];
  const int key = tid & (ATT_KEYS - 1);
  float sk = 0.f;
  if (blk) {
    const int kq = min(key, a.gamma - 1);
#pragma unroll
    for (int p = 0; p < HJ; ++p) sk += a.ssq[(int64_t)((a.nH + kvh) * HJ + p) * a.M + row * a.gamma + kq];
  }
  bf16x8 qh[NS], ql[NS];
  auto prep = [&]() {
    const float r = 1.f / sqrtf(qss / HD + a.eps);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      float t[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        t[e] = qv[s][0][e] * r;
        t[4 + e] = qv[s][1][e] * r;
      }
      split8(t, qh[s], ql[s]);
    }
  };

  f32x4 o[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_part = 0.f;
  if (blk) {
    const int64_t off = ((int64_t)row * a.nKv + kvh) * a.gamma * HD;
    attn_keys<HD, false, NTH, NTW>(a.kb + off, a.vb + off, j0, j1, 1.f / sqrtf(sk / HD + a.eps), prep, qh, ql, o, 0,
                                   m_run, l_part, Ks, Vt);
  } else {
    const int64_t kvoff = (int64_t)kvh * len * HD * (KVB ? 2 : 4);
    const char* vb = (const char*)a.row[row].v + kvoff;
    if constexpr (VO) {
      const VoCtx vo = vo_setup<HD, VO>(vot, a, row);
      attn_keys<HD, KVB, NTH, NTW, true>(vb, vb, j0, j1, 1.f, prep, qh, ql, o, 0, m_run, l_part, Ks, Vt, vo);
    } else {
      const char* kb = (const char*)a.row[row].k + kvoff;
      attn_keys<HD, KVB, NTH, NTW>(kb, vb, j0, j1, 1.f, prep, qh, ql, o, 0, m_run, l_part, Ks, Vt);
    }
  }

  float l = l_part;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  const int64_t base = ((int64_t)sg * a.nKv + kvh) * a.nq + qr;
  const int64_t grp = ((int64_t)sg * a.nKv + kvh) * (a.nq / 16) + wave;
  store_part<KVB, true, HD>(a.opart, base * HD + 4 * gq, grp * 16 * HD, 0, o, l);
  if (gq == 0) {
    a.ml[base * 2] = m_run;
    a.ml[base * 2 + 1] = l;
  }
}

bool attn_vonly_ok(int nq, int hd, bool wide) {
  const int nth = wide ? 4 * nq : ATT_NTH;
  if (hd != 64 && hd != 128 && hd != 256) return false;
  return (hd / 16) % (nth / ATT_KEYS) == 0 && ATT_KEYS * (hd / 8) % nth == 0;
}

bool attn_wide_ok(int nq, int hd) {
  const int nqt = nq / 16;
  if (nq % 16 != 0 || (nqt != 2 && nqt != 4 && nqt != 8)) return false;
  if (hd != 64 && hd != 128 && hd != 256) return false;
  // at most two staging items per thread (more spill registers)
  const int items = ATT_KEYS * (hd / 8), nth = 64 * nqt;
  return items % nth == 0 && items >= nth && items <= 2 * nth;
}

hipError_t launch_attn_wide(const AttnArgs& a, bool kv_bf16, int nsplit, hipStream_t st) {
  if (!attn_wide_ok(a.nq, a.hd)) return hipErrorInvalidValue;
  const dim3 grid(nsplit, a.nKv);  // nsplit: the split count, or 8 * slots per XCD (xcd_rows)
  const int nqt = a.nq / 16;
#define DSP_WIDE(H, Q)                                                                                    \
  if (a.vonly) {                                                                                          \
    if constexpr (vo_layout_ok<H, 64 * Q>()) {                                                            \
      if (!kv_bf16) return hipErrorInvalidValue;                                                          \
      hipLaunchKernelGGL((k_attn_wide<H, true, Q, true>), grid, dim3(64 * Q), 0, st, a);                  \
    } else {                                                                                              \
      return hipErrorInvalidValue;                                                                        \
    }                                                                                                     \
  } else if (kv_bf16) hipLaunchKernelGGL((k_attn_wide<H, true, Q, false>), grid, dim3(64 * Q), 0, st, a); \
  else hipLaunchKernelGGL((k_attn_wide<H, false, Q, false>), grid, dim3(64 * Q), 0, st, a);
  if (a.hd == 64) {
    if (nqt == 2) { DSP_WIDE(64, 2) }
    else { DSP_WIDE(64, 4) }
  } else if (a.hd == 128) {
    if (nqt == 4) { DSP_WIDE(128, 4) }
    else { DSP_WIDE(128, 8) }
  } else { DSP_WIDE(256, 8) }
#undef DSP_WIDE
  return hipGetLastError();
}

hipError_t launch_attn(const AttnArgs& a, bool kv_bf16, int nsplit, hipStream_t st) {
  dim3 grid(nsplit, a.nKv, (a.nq + 15) / 16), block(ATT_NTH);
#define DSP_ATTN(H)                                                                            \
  if (a.vonly) {                                                                               \
    if constexpr (vo_layout_ok<H, ATT_NTH>()) {                                                \
      if (!kv_bf16) return hipErrorInvalidValue;                                               \
      hipLaunchKernelGGL((k_attn<H, true, true>), grid, block, 0, st, a);                      \
    } else {                                                                                   \
      return hipErrorInvalidValue;                                                             \
    }                                                                                          \
  } else if (kv_bf16) hipLaunchKernelGGL((k_attn<H, true, false>), grid, block, 0, st, a);     \
  else hipLaunchKernelGGL((k_attn<H, false, false>), grid, block, 0, st, a);
  if (a.hd == 64) { DSP_ATTN(64) }
  else if (a.hd == 128) { DSP_ATTN(128) }
  else { DSP_ATTN(256) }
#undef DSP_ATTN
  return hipGetLastError();
}

}  // namespace dsp
