// Weight-streaming GEMM y = x . W^T on bf16 MFMA (v_mfma_f32_16x16x32_bf16).
//
// Used for every linear layer of the drafter (deepspec.ts, matmulW: x @ W^T
// with W kept in its [out, in] storage): q|k, o, gate|up, down, lm_head, fc
// and the per-layer k_proj of the context projection.
//
// Work split: a 256-thread workgroup = 4 wave64s; wave w owns one 16-column
// output tile (blockIdx.x*4 + w) and the workgroup owns one K slice
// (blockIdx.y) and one block of MT*16 rows (blockIdx.z).  Each wave issues all
// weight loads of a K sub-slice straight from HBM into registers first (16 B
// per lane per 32-wide k step, the B operand layout needs no shuffling), then
// the workgroup stages the activation sub-slice into LDS already split into
// bf16 hi + lo halves in A-operand order, and the MFMAs run hi and lo against
// the same weight registers.  Activations are fp32 in HBM; hi + lo carries
// ~16 mantissa bits, which the draft round needs (scale-1 attention amplifies
// input rounding).  bf16 inputs (the X-is-bf16 variant) are exact in hi.
//
// Weight kinds:
//   bf16: used as is.
//   f32 : split hi + lo as well; x_hi*w_hi + x_lo*w_hi + x_hi*w_lo.
//   q4  : affine 4-bit, groups of 64 along K.  Codes become the exact bf16
//         values 1 + q/16 with two bit operations per pair, and
//         sum_k x (s q + b) = 16 s * sum x (1 + q/16) + (b - 16 s) * sum x
//         is applied per group after the group's MFMAs (sum x per row and
//         group comes from the staging pass), so no dequantised weight is
//         ever rounded.
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

template <int WK, bool XBF, int MT>
__global__ __launch_bounds__(256) void k_gemm(const GemmArgs g) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int KCMAX = (WK == WK_F32) ? 256 : 512;
  constexpr int SMAX = KCMAX / 32;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, gq = lane >> 4;
  const int KC = g.kc;
  const int nfull = KC >> 5;
  const int ngmax = KC >> 6;
  u32x4* xhi = (u32x4*)smem;
  u32x4* xlo = xhi + MT * nfull * 64;
  float* xsum = (float*)(xhi + (XBF ? 1 : 2) * MT * nfull * 64);

  const int nt = blockIdx.x * 4 + wave;
  const bool active = nt * 16 < g.N;
  int si = 0;
  for (int i = 1; i < g.nseg; ++i)
    if (nt * 16 >= g.seg[i].n0) si = i;
  const int64_t wrow = (int64_t)(nt * 16 - g.seg[si].n0 + (lane & 15));
  const int mbase = blockIdx.z * (MT * 16);
  const int kbeg = blockIdx.y * g.kslice;
  const int kend = min(g.K, kbeg + g.kslice);

  f32x4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int kc = kbeg; kc < kend; kc += KC) {
    const int klen = min(KC, kend - kc);
    const int nsteps = klen >> 5;

    // 1. weights of this sub-slice -> registers
    u32x4 wv[WK == WK_F32 ? 2 * SMAX : (WK == WK_BF16 ? SMAX : 1)];
    u32x2 wq[WK == WK_Q4 ? SMAX / 2 : 1];
    float qs[WK == WK_Q4 ? SMAX / 2 : 1], qb[WK == WK_Q4 ? SMAX / 2 : 1];
    if (active) {
      if constexpr (WK == WK_BF16) {
        const uint16_t* p = (const uint16_t*)g.seg[si].w + wrow * g.K + kc + 8 * gq;
#pragma unroll
        for (int s = 0; s < SMAX; ++s)
          if (s < nsteps) wv[s] = *(const u32x4*)(p + 32 * s);
      } else if constexpr (WK == WK_F32) {
        const float* p = (const float*)g.seg[si].w + wrow * g.K + kc + 8 * gq;
#pragma unroll
        for (int s = 0; s < SMAX; ++s)
          if (s < nsteps) {
            wv[2 * s] = *(const u32x4*)(p + 32 * s);
            wv[2 * s + 1] = *(const u32x4*)(p + 32 * s + 4);
          }
      } else {
        const uint32_t* p = (const uint32_t*)g.seg[si].w + wrow * (g.K >> 3) + (kc >> 3) + 2 * gq;
        const uint16_t* ps = (const uint16_t*)g.seg[si].s + wrow * (g.K >> 6) + (kc >> 6);
        const uint16_t* pb = (const uint16_t*)g.seg[si].b + wrow * (g.K >> 6) + (kc >> 6);
#pragma unroll
        for (int j = 0; j < SMAX / 2; ++j)
          if (2 * j < nsteps) {
            wq[j] = *(const u32x2*)(p + 8 * j);
            qs[j] = bf2f(ps[j]);
            qb[j] = bf2f(pb[j]);
          }
      }
    }

    // 2. activation sub-slice -> LDS (hi / lo planes, A-operand order)
    if constexpr (WK == WK_Q4) {
      for (int i = tid; i < MT * 16 * ngmax; i += 256) xsum[i] = 0.f;
      __syncthreads();
    }
    const int kq = klen >> 3;
    for (int it = tid; it < MT * 16 * kq; it += 256) {
      const int ml = it / kq, k8 = it - ml * kq;
      const int m = mbase + ml;
      float v[8];
      if (m < g.M) {
        if constexpr (XBF) {
          u32x4 r = *(const u32x4*)((const uint16_t*)g.X + (int64_t)m * g.ldx + kc + 8 * k8);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[2 * e] = __uint_as_float(r[e] << 16);
            v[2 * e + 1] = __uint_as_float(r[e] & 0xFFFF0000u);
          }
        } else {
          const float* px = (const float*)g.X + (int64_t)m * g.ldx + kc + 8 * k8;
          f32x4 a = *(const f32x4*)px, b = *(const f32x4*)(px + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) { v[e] = a[e]; v[4 + e] = b[e]; }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = 0.f;
      }
      int s, qg;
      float e8[8];
      if constexpr (WK == WK_Q4) {
        const int grp = k8 >> 3, r = k8 & 7;
        qg = r >> 1;
        s = 2 * grp + (r & 1);
        const int perm[8] = {0, 4, 1, 5, 2, 6, 3, 7};
        float sum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) { e8[e] = v[perm[e]]; sum += v[e]; }
        atomicAdd(&xsum[ml * ngmax + grp], sum);
      } else {
        s = k8 >> 2;
        qg = k8 & 3;
#pragma unroll
        for (int e = 0; e < 8; ++e) e8[e] = v[e];
      }
      const int slot = ((ml >> 4) * nfull + s) * 64 + qg * 16 + (ml & 15);
      if constexpr (XBF) {
        xhi[slot] = __builtin_bit_cast(u32x4, to_bf16x8(e8));
      } else {
        bf16x8 h, l;
        split8(e8, h, l);
        xhi[slot] = __builtin_bit_cast(u32x4, h);
        xlo[slot] = __builtin_bit_cast(u32x4, l);
      }
    }
    __syncthreads();

    // 3. MFMAs
    if (active) {
      if constexpr (WK == WK_BF16) {
#pragma unroll
        for (int s = 0; s < SMAX; ++s)
          if (s < nsteps) {
            const bf16x8 w = __builtin_bit_cast(bf16x8, wv[s]);
#pragma unroll
            for (int t = 0; t < MT; ++t) {
              const int o = (t * nfull + s) * 64 + lane;
              acc[t] = mfma16(__builtin_bit_cast(bf16x8, xhi[o]), w, acc[t]);
              if constexpr (!XBF) acc[t] = mfma16(__builtin_bit_cast(bf16x8, xlo[o]), w, acc[t]);
            }
          }
      } else if constexpr (WK == WK_F32) {
#pragma unroll
        for (int s = 0; s < SMAX; ++s)
          if (s < nsteps) {
            float w8[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              w8[e] = __uint_as_float(wv[2 * s][e]);
              w8[4 + e] = __uint_as_float(wv[2 * s + 1][e]);
            }
            bf16x8 wh, wl;
            split8(w8, wh, wl);
#pragma unroll
            for (int t = 0; t < MT; ++t) {
              const int o = (t * nfull + s) * 64 + lane;
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
              const bf16x8 w = q4_decode(wq[j][sub]);
#pragma unroll
              for (int t = 0; t < MT; ++t) {
                const int o = (t * nfull + 2 * j + sub) * 64 + lane;
                tmp[t] = mfma16(__builtin_bit_cast(bf16x8, xhi[o]), w, tmp[t]);
                if constexpr (!XBF) tmp[t] = mfma16(__builtin_bit_cast(bf16x8, xlo[o]), w, tmp[t]);
              }
            }
            const float sc = 16.f * qs[j], bc = qb[j] - sc;
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                acc[t][i] += sc * tmp[t][i] + bc * xsum[(t * 16 + 4 * gq + i) * ngmax + j];
          }
      }
    }
    __syncthreads();
  }

  // 4. partial tile -> P[blockIdx.y]
  if (active) {
    float* out = g.P + (int64_t)blockIdx.y * g.M * g.N;
    const int n = nt * 16 + (lane & 15);
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = mbase + t * 16 + 4 * gq + i;
        if (m < g.M) out[(int64_t)m * g.N + n] = acc[t][i];
      }
  }
}

size_t gemm_lds_bytes(int wkind, bool x_bf16, int mt, int kc) {
  size_t b = (size_t)mt * (kc / 32) * 64 * 16 * (x_bf16 ? 1 : 2);
  if (wkind == WK_Q4) b += (size_t)mt * 16 * (kc / 64) * 4;
  return b;
}

template <int WK, bool XBF>
static hipError_t launch_mt(const GemmArgs& a, int mt, int S, hipStream_t st) {
  const int mblocks = (a.M + mt * 16 - 1) / (mt * 16);
  dim3 grid((a.N / 16 + 3) / 4, S, mblocks);
  const size_t lds = gemm_lds_bytes(WK, XBF, mt, a.kc);
  switch (mt) {
    case 1: hipLaunchKernelGGL((k_gemm<WK, XBF, 1>), grid, dim3(256), lds, st, a); break;
    case 2: hipLaunchKernelGGL((k_gemm<WK, XBF, 2>), grid, dim3(256), lds, st, a); break;
    case 3: hipLaunchKernelGGL((k_gemm<WK, XBF, 3>), grid, dim3(256), lds, st, a); break;
    default: hipLaunchKernelGGL((k_gemm<WK, XBF, 4>), grid, dim3(256), lds, st, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& a, int wkind, bool x_bf16, int mt, int S, hipStream_t st) {
  if (wkind == WK_BF16) return x_bf16 ? launch_mt<WK_BF16, true>(a, mt, S, st) : launch_mt<WK_BF16, false>(a, mt, S, st);
  if (wkind == WK_F32) return x_bf16 ? launch_mt<WK_F32, true>(a, mt, S, st) : launch_mt<WK_F32, false>(a, mt, S, st);
  return x_bf16 ? launch_mt<WK_Q4, true>(a, mt, S, st) : launch_mt<WK_Q4, false>(a, mt, S, st);
}

}  // namespace dsp
