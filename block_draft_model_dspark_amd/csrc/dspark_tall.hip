// Tiled bf16 MFMA GEMM for many activation rows.
//
// The weight-streaming GEMM (dspark_gemm.hip) gives each workgroup one or
// two 16-row tiles and streams the weights once per row block: right for the
// 16-row draft block, wasteful once there are hundreds of rows (a batch of
// draft rows, or a long context to project), where the same weight tile is
// fetched again for every row block and the work is bound by MFMA rate, not
// by HBM.  For those shapes the product is formed here in three steps:
//   1. k_xprep: the input rows as bf16 planes.  fp32 rows (and normed
//      residual rows, formed from the stored row statistics exactly as the
//      weight-streaming kernel forms them) become a hi and a lo plane whose
//      sum carries the fp32 value; bf16 input rows are used as they are.
//   2. k_tall: T[m, n] = sum over planes of X_p[m, :] . W[n, :] in fp32,
//      BM x BN output tiles, both operands staged through LDS in 64-wide K
//      steps (the global loads of the next one or two steps in flight during
//      this step's MFMAs), four waves of (BM/2) x (BN/2).  Few output tiles split
//      K over blockIdx.z into partial planes that the epilogue adds.
//   3. the GEMM's own epilogue (norm statistics, q|k RoPE, GELU gate, logit
//      softcap, context K/V) reads T: k_gemm_epi / k_kv_epi.
#include "dspark_kernels.hpp"
#include "dspark_common.hpp"

namespace dsp {

// ---------------------------------------------------------------------------
// 1. input rows -> bf16 hi / lo planes [2][M][K] (plane stride t.plane)
// ---------------------------------------------------------------------------
// One workgroup per row.  XM_NORM: deepspec.ts, #forwardBackbone sandwich
// norms; hn = (h + rms(y) * w1 * y) * sc, x = rms(hn) * w2 (x = hn without
// w2), the RMS factors taken from the 64-column statistics (see NormIn), and
// hn written to hout when it is given.
template <int XM>
__global__ __launch_bounds__(256) void k_xprep(const GemmArgs g, uint16_t* xop, int64_t plane) {
  __shared__ RowStats red[4];
  const int m = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = g.K;
  float r1 = 1.f, r2 = 1.f, sc = 1.f;
  if constexpr (XM == XM_NORM) {
    const NormIn& n = g.nin;
    RowStats s = {0.0, 0.0, 0.0, 0.0};
    for (int p = tid; p < n.nparts; p += 256) {
      const RowStats v = n.sums[(int64_t)p * g.M + m];
      s.x += v.x;
      s.y += v.y;
      s.z += v.z;
      s.w += v.w;
    }
    s.x = wave_sum_d(s.x);
    s.y = wave_sum_d(s.y);
    s.z = wave_sum_d(s.z);
    s.w = wave_sum_d(s.w);
    if (lane == 0) red[wave] = s;
    __syncthreads();
    s = red[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      s.x += red[w].x;
      s.y += red[w].y;
      s.z += red[w].z;
      s.w += red[w].w;
    }
    sc = n.sc ? *n.sc : 1.f;
    const float2 f = norm_factors(s, sc, K, n.eps);
    r1 = f.x;
    r2 = f.y;
  }
  for (int k8 = tid; k8 < (K >> 3); k8 += 256) {
    const int k = 8 * k8;
    float v[8];
    if constexpr (XM == XM_NORM) {
      const NormIn& n = g.nin;
      const bool bf = n.act_bf16 != 0;
      float h[8], y[8], w1[8], w2[8];
      const float* ph = n.h ? n.h : n.y;
      const float* py = n.y ? n.y : n.h;
      const f32x4 h0 = *(const f32x4*)(ph + (int64_t)m * n.ld + k), h1 = *(const f32x4*)(ph + (int64_t)m * n.ld + k + 4);
      const f32x4 y0 = *(const f32x4*)(py + (int64_t)m * n.ld + k), y1 = *(const f32x4*)(py + (int64_t)m * n.ld + k + 4);
      const void* p1 = n.y ? n.w1 : n.w2;
      const void* p2 = n.w2 ? n.w2 : p1;
      cvt_act8(ld_act8(p1, k, bf), bf, w1);
      cvt_act8(ld_act8(p2, k, bf), bf, w2);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        h[q] = h0[q];
        h[4 + q] = h1[q];
        y[q] = y0[q];
        y[4 + q] = y1[q];
      }
      float hn[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float hv = n.h ? h[q] : 0.f;
        const float yv = n.y ? y[q] * r1 * w1[q] : 0.f;
        hn[q] = (hv + yv) * sc;
        v[q] = n.w2 ? hn[q] * r2 * w2[q] : hn[q];
      }
      if (n.hout) {
        float* dst = n.hout + (int64_t)m * n.ld + k;
        *(f32x4*)dst = f32x4{hn[0], hn[1], hn[2], hn[3]};
        *(f32x4*)(dst + 4) = f32x4{hn[4], hn[5], hn[6], hn[7]};
      }
    } else {
      const float* px = (const float*)g.X + (int64_t)m * g.ldx + k;
      const f32x4 a = *(const f32x4*)px, b = *(const f32x4*)(px + 4);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[q] = a[q];
        v[4 + q] = b[q];
      }
    }
    bf16x8 hi, lo;
    split8(v, hi, lo);
    *(u32x4*)(xop + (int64_t)m * K + k) = __builtin_bit_cast(u32x4, hi);
    *(u32x4*)(xop + plane + (int64_t)m * K + k) = __builtin_bit_cast(u32x4, lo);
  }
}

// ---------------------------------------------------------------------------
// 1b. split-K epilogue of o / down fused with the next input preparation
//     (deepspec.ts, #forwardBackbone sandwich norms): one workgroup per row,
//     eight columns per thread and item
// ---------------------------------------------------------------------------
constexpr int SP_IT = SP_KMAX / 8 / 256;  // items per thread

__device__ __forceinline__ double block_sum_d(double v, double* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum_d(v);
  __syncthreads();  // the previous use of red is complete
  if (lane == 0) red[wave] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

__global__ __launch_bounds__(256) void k_sums_prep(const SumsPrepArgs a) {
  __shared__ double red[4];
  const int m = blockIdx.x, tid = threadIdx.x;
  const int nk8 = a.K >> 3;
  const bool bf = a.act_bf16 != 0;
  float y[SP_IT][8], hn[SP_IT][8];
  // 1. y = sum of the slices, and sum y^2
  double syy = 0.0;
#pragma unroll
  for (int it = 0; it < SP_IT; ++it) {
    const int k = 8 * (tid + 256 * it);
#pragma unroll
    for (int q = 0; q < 8; ++q) y[it][q] = 0.f;
    if (k < a.K) {
      const float* tp = a.T + (int64_t)m * a.ldt + k;
      for (int s = 0; s < a.S; ++s) {
        const f32x4 p0 = *(const f32x4*)(tp + s * a.tstride), p1 = *(const f32x4*)(tp + s * a.tstride + 4);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          y[it][q] += p0[q];
          y[it][4 + q] += p1[q];
        }
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) syy += (double)y[it][q] * y[it][q];
    }
  }
  const float r1 = (float)(1.0 / sqrt(block_sum_d(syy, red) / a.K + (double)a.eps));
  const float sc = a.sc ? *a.sc : 1.f;
  // 2. hn = (h + r1 w1 y) sc, and sum hn^2
  double shh = 0.0;
#pragma unroll
  for (int it = 0; it < SP_IT; ++it) {
    const int k = 8 * (tid + 256 * it);
    if (k < a.K) {
      float w1[8];
      cvt_act8(ld_act8(a.w1, k, bf), bf, w1);
      f32x4 h0 = f32x4{0.f, 0.f, 0.f, 0.f}, h1 = h0;
      if (a.h) {
        const float* hp = a.h + (int64_t)m * a.ldh + k;
        h0 = *(const f32x4*)hp;
        h1 = *(const f32x4*)(hp + 4);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float hv = q < 4 ? h0[q] : h1[q - 4];
        hn[it][q] = (hv + y[it][q] * r1 * w1[q]) * sc;
        shh += (double)hn[it][q] * hn[it][q];
      }
      if (a.hout) {
        float* dst = a.hout + (int64_t)m * a.ldh + k;
        *(f32x4*)dst = f32x4{hn[it][0], hn[it][1], hn[it][2], hn[it][3]};
        *(f32x4*)(dst + 4) = f32x4{hn[it][4], hn[it][5], hn[it][6], hn[it][7]};
      }
    }
  }
  const float r2 = (float)(1.0 / sqrt(block_sum_d(shh, red) / a.K + (double)a.eps));
  // 3. x = hn r2 w2 as hi / lo planes
#pragma unroll
  for (int it = 0; it < SP_IT; ++it) {
    const int k = 8 * (tid + 256 * it);
    if (k < a.K) {
      float v[8];
      if (a.w2) {
        float w2[8];
        cvt_act8(ld_act8(a.w2, k, bf), bf, w2);
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = hn[it][q] * r2 * w2[q];
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = hn[it][q];
      }
      bf16x8 hi, lo;
      split8(v, hi, lo);
      *(u32x4*)(a.xop + (int64_t)m * a.K + k) = __builtin_bit_cast(u32x4, hi);
      *(u32x4*)(a.xop + a.plane + (int64_t)m * a.K + k) = __builtin_bit_cast(u32x4, lo);
    }
  }
}

// ---------------------------------------------------------------------------
// 2. T = sum_p X_p W^T, BM x BN tiles, K steps of 64
// ---------------------------------------------------------------------------
constexpr int TBK = 64;  // K step

// Two forms, by the number of input planes:
//  - two planes (hi + lo): two steps of global loads in flight in registers,
//    rows padded to a 160-byte LDS pitch (of the 144, 160, 176 and 208-byte
//    pitches the MFMA operand reads stall least at this one), 60 KB of LDS
//    and ~200 VGPRs: two workgroups per CU;
//  - one plane: one step in flight, 128-byte rows with their 16-byte chunks
//    xor-swizzled by row (operand reads spread over the banks without
//    padding), 32 KB of LDS and ~126 VGPRs: four workgroups per CU, whose
//    waves hide each other's waits (the two-plane kernel in this form, at
//    three workgroups per CU, ran 4-8% slower than in the first).
template <int NP>
struct TallForm {
  static constexpr bool one = NP == 1;
  static constexpr int LD = one ? TBK : TBK + 16;  // LDS row pitch (bf16)
  __device__ static constexpr int chunk(int row, int c) { return one ? (c ^ (row & 7)) : c; }
};

template <int BM, int BN, int NP>
__global__ __launch_bounds__(256, NP == 1 ? 3 : 2) void k_tall(const TallArgs t) {
  using F = TallForm<NP>;
  constexpr int TLD = F::LD;
  constexpr int WM = BM / 2, WN = BN / 2, FM = WM / 16, FN = WN / 16;
  constexpr int AIT = BM * (TBK / 8) / 256, BIT = BN * (TBK / 8) / 256;  // 16-byte items per thread
  static_assert(AIT >= 1 && BIT >= 1, "tile too small for 256 threads");
  __shared__ __align__(16) uint16_t As[NP][BM * TLD];
  __shared__ __align__(16) uint16_t Bs[BN * TLD];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, ln = lane & 15, gq = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  // tile order: see tall_tile_of (XCD-aware renumbering of the grid)
  int bx, by;
  tall_tile_of(gridDim.x, gridDim.y, blockIdx.x + gridDim.x * blockIdx.y, bx, by);
  const int m0 = by * BM, n0 = bx * BN;
  const int kb = blockIdx.z * t.kslice, ke = min(t.K, kb + t.kslice);  // this slice of K (multiples of 64)

  // this thread's rows of the two tiles (clamped: rows past M or N repeat
  // the last one and are never stored) and the weight segment of each
  const uint16_t* ap[AIT];
  const uint16_t* bp[BIT];
#pragma unroll
  for (int j = 0; j < AIT; ++j) {
    const int it = tid + 256 * j, r = it >> 3, c8 = it & 7;
    ap[j] = t.X + (int64_t)min(m0 + r, t.M - 1) * t.ldx + 8 * c8;
  }
#pragma unroll
  for (int j = 0; j < BIT; ++j) {
    const int it = tid + 256 * j, r = it >> 3, c8 = it & 7;
    // gate|up pairing: tile rows 0..63 are gate rows 64x.., 64..127 up rows
    const int n = (BN == 128 && t.gelu) ? (r < 64 ? 64 * bx + r : t.N / 2 + 64 * bx + r - 64)
                                        : min(n0 + r, t.N - 1);
    // segment lookup with uniform (scalar) reads of the argument array
    const void* w = t.seg[0].w;
    int nb = t.seg[0].n0;
#pragma unroll
    for (int i = 1; i < MAX_SEG; ++i) {
      const void* wi = t.seg[i].w;
      const int ni = t.seg[i].n0;
      const bool in = i < t.nseg && n >= ni;
      w = in ? wi : w;
      nb = in ? ni : nb;
    }
    bp[j] = (const uint16_t*)w + (int64_t)(n - nb) * t.K + 8 * c8;
  }
  // register sets of global loads in flight: two planes, steps k and k + 64
  // load while step k - 64 is multiplied; one plane, step k while k - 64 is
  // (a step past the slice reloads the slice's last one, so every thread
  // always has the same loads in flight)
  struct Stage {
    u32x4 a[NP][AIT], b[BIT];
  };
  Stage st0, st1;
  auto load = [&](Stage& r, int k0) {
    k0 = min(k0, ke - TBK);
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int j = 0; j < AIT; ++j) r.a[p][j] = *(const u32x4*)(ap[j] + p * t.plane + k0);
#pragma unroll
    for (int j = 0; j < BIT; ++j) r.b[j] = *(const u32x4*)(bp[j] + k0);
  };
  auto store = [&](const Stage& r) {
#pragma unroll
    for (int j = 0; j < AIT; ++j) {
      const int it = tid + 256 * j, rr = it >> 3, c8 = it & 7;
#pragma unroll
      for (int p = 0; p < NP; ++p) *(u32x4*)&As[p][rr * TLD + 8 * F::chunk(rr, c8)] = r.a[p][j];
    }
#pragma unroll
    for (int j = 0; j < BIT; ++j) {
      const int it = tid + 256 * j, rr = it >> 3, c8 = it & 7;
      *(u32x4*)&Bs[rr * TLD + 8 * F::chunk(rr, c8)] = r.b[j];
    }
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto step = [&]() {
#pragma unroll
    for (int s = 0; s < TBK / 32; ++s) {
      bf16x8 bfr[FN];
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = __builtin_bit_cast(bf16x8, *(const u32x4*)&Bs[(WN * wn + 16 * j + ln) * TLD + 8 * F::chunk(ln, 4 * s + gq)]);
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const bf16x8 afr =
              __builtin_bit_cast(bf16x8, *(const u32x4*)&As[p][(WM * wm + 16 * i + ln) * TLD + 8 * F::chunk(ln, 4 * s + gq)]);
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] = mfma16(afr, bfr[j], acc[i][j]);
        }
    }
  };
  if constexpr (F::one) {
    load(st0, kb);
    for (int k0 = kb; k0 < ke; k0 += TBK) {
      __syncthreads();  // every wave is done reading the previous step
      store(st0);
      __syncthreads();
      load(st0, k0 + TBK);
      step();
    }
  } else {
    load(st0, kb);
    load(st1, kb + TBK);
    int k0 = kb;
    for (; k0 + 2 * TBK <= ke; k0 += 2 * TBK) {
      __syncthreads();  // every wave is done reading the previous step
      store(st0);
      __syncthreads();
      load(st0, k0 + 2 * TBK);
      step();
      __syncthreads();
      store(st1);
      __syncthreads();
      load(st1, k0 + 3 * TBK);
      step();
    }
    if (k0 < ke) {  // an odd last step (uniform)
      __syncthreads();
      store(st0);
      __syncthreads();
      step();
    }
  }
  float* const T = t.T + blockIdx.z * t.tstride;

  if constexpr (WN == 64 && NP == 2) {
    if (t.gelu) {  // uniform: waves wn = 1 hold the up columns of the gate columns of waves wn = 0
      float* ex = (float*)&As[0][0];  // 2 x 64 x 64 floats (32 KiB) of the staging planes
      __syncthreads();                // every wave is done with the last step's operands
      if (wn == 1)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) ex[(wm * 64 + 16 * i + 4 * gq + q) * 64 + 16 * j + ln] = acc[i][j][q];
      __syncthreads();
      if (wn == 0)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = 16 * i + 4 * gq + q, m = m0 + WM * wm + r;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
              const int c = 16 * j + ln;
              float* xe = &ex[(wm * 64 + r) * 64 + c];
              const float x = gelu_tanh(acc[i][j][q]) * *xe;
              if (t.act_planes) *xe = x;  // (this thread's own element)
              else if (m < t.M) t.act[(int64_t)m * t.ld_act + 64 * bx + c] = x;
            }
          }
      if (t.act_planes) {
        // the 128 x 64 products as hi / lo planes, eight columns (16 bytes) per store
        __syncthreads();
        const int64_t I = t.N / 2;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int idx = tid + 256 * k, rr = idx >> 3, c8 = idx & 7;  // rr: row of the 128-row tile
          const int m = m0 + rr;
          if (m < t.M) {
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = ex[rr * 64 + 8 * c8 + e];
            bf16x8 hi, lo;
            split8(v, hi, lo);
            uint16_t* dst = t.act_planes + (int64_t)m * I + 64 * bx + 8 * c8;
            *(u32x4*)dst = __builtin_bit_cast(u32x4, hi);
            *(u32x4*)(dst + t.act_plane) = __builtin_bit_cast(u32x4, lo);
          }
        }
      }
      return;
    }
  }
  if constexpr (WN == 64) {
    if (t.lm) {  // uniform: the wave's 64 columns are one walk chunk
      const int nc0 = n0 + WN * wn;
      float b[FN];
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int n = min(nc0 + 16 * j + ln, t.N - 1);
        b[j] = t.aux ? walk_bound(t.aux, n, t.N) : 0.f;
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int m = m0 + WM * wm + 16 * i + 4 * gq + q;
          float lo = -INFINITY, hi = -INFINITY;
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const int n = nc0 + 16 * j + ln;
            float z = acc[i][j][q];
            if (t.cap > 0.f) z = t.cap * tanh_fast(z / t.cap);
            if (n < t.N) {
              if (m < t.M) T[(int64_t)m * t.ldt + n] = z;
              lo = fmaxf(lo, z - b[j]);
              hi = fmaxf(hi, z + b[j]);
            }
          }
          lo = row16_max(lo);
          hi = row16_max(hi);
          if (ln == 0 && m < t.M && nc0 < t.N) t.lohi[(int64_t)m * t.NC + nc0 / 64] = make_float2(lo, hi);
        }
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = n0 + WN * wn + 16 * j + ln;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = m0 + WM * wm + 16 * i + 4 * gq + q;
        if (m < t.M && n < t.N) T[(int64_t)m * t.ldt + n] = acc[i][j][q];
      }
    }
}

hipError_t launch_xprep(const GemmArgs& g, int xmode, uint16_t* xop, int64_t plane, hipStream_t st) {
  if (xmode == XM_NORM) {
    if (g.nin.nparts * 64 != g.K) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_xprep<XM_NORM>, dim3(g.M), dim3(256), 0, st, g, xop, plane);
  } else if (xmode == XM_F32) {
    hipLaunchKernelGGL(k_xprep<XM_F32>, dim3(g.M), dim3(256), 0, st, g, xop, plane);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_sums_prep(const SumsPrepArgs& a, hipStream_t st) {
  if (a.K <= 0 || a.K > SP_KMAX || a.K % 8 != 0 || a.S < 1 || a.M < 1 || !a.T || !a.w1 || !a.xop)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_sums_prep, dim3(a.M), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_tall(const TallArgs& t, int tile, int np, int S, hipStream_t st) {
  if (t.K % TBK != 0 || t.kslice % TBK != 0 || t.kslice <= 0 || (int64_t)S * t.kslice < t.K ||
      (int64_t)(S - 1) * t.kslice >= t.K || t.M <= 0 || t.N <= 0 || t.nseg < 1 || t.nseg > MAX_SEG)
    return hipErrorInvalidValue;
  // the fused logits need whole 64-entry chunks per wave (128 x 128 tiles)
  // and the final product (one K slice)
  if (t.lm && (tile != TALL_128 || S != 1 || t.N % 64 != 0 || !t.lohi || t.ldt != t.N)) return hipErrorInvalidValue;
  // the fused gate|up pairs 64 gate with 64 up columns per tile
  if (t.gelu && (tile != TALL_128 || S != 1 || np != 2 || t.N % 128 != 0 || !t.act || t.lm)) return hipErrorInvalidValue;
  const int bm = tile == TALL_128 ? 128 : 64, bn = bm;
  const dim3 grid((t.N + bn - 1) / bn, (t.M + bm - 1) / bm, S);
  if (tile == TALL_128) {
    if (np == 1) hipLaunchKernelGGL((k_tall<128, 128, 1>), grid, dim3(256), 0, st, t);
    else hipLaunchKernelGGL((k_tall<128, 128, 2>), grid, dim3(256), 0, st, t);
  } else {
    if (np == 1) hipLaunchKernelGGL((k_tall<64, 64, 1>), grid, dim3(256), 0, st, t);
    else hipLaunchKernelGGL((k_tall<64, 64, 2>), grid, dim3(256), 0, st, t);
  }
  return hipGetLastError();
}

}  // namespace dsp
