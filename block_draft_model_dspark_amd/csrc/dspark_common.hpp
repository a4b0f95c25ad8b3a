// Shared device helpers for the gfx950 DSpark kernels: bf16 conversion, the
// hi/lo bf16 split that carries fp32 activations through bf16 MFMA, the
// 16x16x32 bf16 MFMA, and wave64 reductions.
//
// MFMA operand layout (v_mfma_f32_16x16x32_bf16, wave64), lane l, g = l >> 4:
//   A (16 rows x 32 k): row l & 15, k = 8g .. 8g+7 (eight bf16)
//   B (32 k x 16 cols): col l & 15, k = 8g .. 8g+7
//   D (16 x 16 f32):    col l & 15, rows 4g .. 4g+3
// Any permutation of k applied identically to A and B leaves D unchanged; the
// kernels use that freedom to match operands to natural memory order.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ uint16_t f2bf(float f) {
  __bf16 b = (__bf16)f;  // round to nearest even (v_cvt_pk_bf16_f32)
  return __builtin_bit_cast(uint16_t, b);
}

// load one activation/norm element stored as f32 (bf16 == false) or bf16
__device__ __forceinline__ float ld_act(const void* p, int64_t i, bool bf16) {
  return bf16 ? bf2f(((const uint16_t*)p)[i]) : ((const float*)p)[i];
}
// The same with one 4-byte load whatever the dtype (for vectors of even
// length), so that the conversion happens after the load is issued and a
// run of such loads stays in flight together.
__device__ __forceinline__ float ld_act_v(const void* p, int64_t i, bool bf16) {
  const uint32_t w = *(const uint32_t*)((const char*)p + (bf16 ? (i >> 1) * 4 : i * 4));
  return __uint_as_float(bf16 ? ((i & 1) ? (w & 0xFFFF0000u) : (w << 16)) : w);
}
// eight consecutive act-dtype values from index k (k % 8 == 0), raw words
struct Raw8 {
  u32x4 a, b;
};
__device__ __forceinline__ Raw8 ld_act8(const void* p, int64_t k, bool bf16) {
  // two 16-byte loads either way (the second repeats the first for bf16), so
  // no branch holds a load whose result must be waited for
  const char* pa = (const char*)p + k * (bf16 ? 2 : 4);
  Raw8 r;
  r.a = *(const u32x4*)pa;
  r.b = *(const u32x4*)(pa + (bf16 ? 0 : 16));
  return r;
}
// one act-dtype element as raw bits (converted later by cvt_act_raw)
__device__ __forceinline__ uint32_t ld_act_raw(const void* p, int64_t i, bool bf16) {
  return bf16 ? (uint32_t)((const uint16_t*)p)[i] : ((const uint32_t*)p)[i];
}
__device__ __forceinline__ float cvt_act_raw(uint32_t r, bool bf16) { return __uint_as_float(bf16 ? r << 16 : r); }
__device__ __forceinline__ void cvt_act8(const Raw8& r, bool bf16, float* v) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (bf16) {
      v[2 * q] = __uint_as_float(r.a[q] << 16);
      v[2 * q + 1] = __uint_as_float(r.a[q] & 0xFFFF0000u);
    } else {
      v[q] = __uint_as_float(r.a[q]);
      v[4 + q] = __uint_as_float(r.b[q]);
    }
  }
}
__device__ __forceinline__ void st_act(void* p, int64_t i, float v, bool bf16) {
  if (bf16) ((uint16_t*)p)[i] = f2bf(v);
  else ((float*)p)[i] = v;
}

// two floats -> packed fp16 pair (round to nearest even)
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  const _Float16 ha = (_Float16)a, hb = (_Float16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}
__device__ __forceinline__ float f16_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// x ~= hi + lo with both bf16: hi = rne(x), lo = rne(x - hi)
__device__ __forceinline__ void split8(const float* v, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __bf16 h = (__bf16)v[i];
    hi[i] = h;
    lo[i] = (__bf16)(v[i] - (float)h);
  }
}
__device__ __forceinline__ bf16x8 to_bf16x8(const float* v) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)v[i];
  return r;
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Cross-lane reductions on DPP (VALU lane moves, no LDS traffic): within a
// row of 16 lanes by quad swaps and row mirrors, across rows by reading one
// lane of each row.  Every lane gets the result.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int DPP_QUAD_1032 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_2301 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int DPP_ROW_MIRROR = 0x140;
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov<DPP_QUAD_1032>(v);
  v += dpp_mov<DPP_QUAD_2301>(v);
  v += dpp_mov<DPP_ROW_HALF_MIRROR>(v);
  v += dpp_mov<DPP_ROW_MIRROR>(v);
  return v;
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_mov<DPP_QUAD_1032>(v));
  v = fmaxf(v, dpp_mov<DPP_QUAD_2301>(v));
  v = fmaxf(v, dpp_mov<DPP_ROW_HALF_MIRROR>(v));
  v = fmaxf(v, dpp_mov<DPP_ROW_MIRROR>(v));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0)) +
      __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16)) +
      __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32)) +
      __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  return fmaxf(fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0)),
                     __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16))),
               fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32)),
                     __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48))));
}
// sum over each half wave (lanes 0..31 and 32..63)
__device__ __forceinline__ float half_sum(float v) {
  v = row16_sum(v);
  const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0)) +
                  __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32)) +
                  __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (threadIdx.x & 32) ? b : a;
}

// fp64 sums over a row of 16 lanes (the same DPP moves on both halves of
// each double) and over the wave (every lane gets the result)
template <int CTRL>
__device__ __forceinline__ double dpp_mov_d(double v) {
  const int2 p = __builtin_bit_cast(int2, v);
  int2 r;
  r.x = __builtin_amdgcn_mov_dpp(p.x, CTRL, 0xF, 0xF, false);
  r.y = __builtin_amdgcn_mov_dpp(p.y, CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, r);
}
__device__ __forceinline__ double row16_sum_d(double v) {
  v += dpp_mov_d<DPP_QUAD_1032>(v);
  v += dpp_mov_d<DPP_QUAD_2301>(v);
  v += dpp_mov_d<DPP_ROW_HALF_MIRROR>(v);
  v += dpp_mov_d<DPP_ROW_MIRROR>(v);
  return v;
}
// Reduce-scatter over the 16 lanes of a row: every lane brings v[0..15] and
// lane l (= lane mod 16) gets the row's sum of v[l].  Four exchange steps
// (partners differ in bit 3, 2, 1, 0 of l: row mirror, half-row mirror, quad
// swaps); at each step a lane keeps the half of its values that its bit
// selects and adds the partner's copy of that half (15 moves and adds
// instead of 16 separate row sums).
__device__ __forceinline__ double row16_reduce_scatter(const double* v) {
  const int l = threadIdx.x & 15;
  double a[8], b[4], c[2];
  {
    const bool up = l & 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] = (up ? v[j + 8] : v[j]) + dpp_mov_d<DPP_ROW_MIRROR>(up ? v[j] : v[j + 8]);
  }
  {
    const bool up = l & 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = (up ? a[j + 4] : a[j]) + dpp_mov_d<DPP_ROW_HALF_MIRROR>(up ? a[j] : a[j + 4]);
  }
  {
    const bool up = l & 2;
#pragma unroll
    for (int j = 0; j < 2; ++j) c[j] = (up ? b[j + 2] : b[j]) + dpp_mov_d<DPP_QUAD_2301>(up ? b[j] : b[j + 2]);
  }
  const bool up = l & 1;
  return (up ? c[1] : c[0]) + dpp_mov_d<DPP_QUAD_1032>(up ? c[0] : c[1]);
}
__device__ __forceinline__ double wave_sum_d(double v) {
  v = row16_sum_d(v);
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// block-wide sum; `red` holds >= blockDim/64 floats; all threads get the result
__device__ __forceinline__ float block_sum(float v, float* red) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, nw = (blockDim.x + 63) >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}
__device__ __forceinline__ float block_max(float v, float* red) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, nw = (blockDim.x + 63) >> 6;
  v = wave_max(v);
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float t = -INFINITY;
  for (int i = 0; i < nw; ++i) t = fmaxf(t, red[i]);
  return t;
}

// (value, index) argmax: larger value wins, lower index on equal values
__device__ __forceinline__ bool better(float u, int i, float bu, int bi) {
  return u > bu || (u == bu && i < bi);
}
__device__ __forceinline__ void wave_argmax(float& u, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float ou = __shfl_xor(u, o);
    int oi = __shfl_xor(i, o);
    if (better(ou, oi, u, i)) { u = ou; i = oi; }
  }
}
__device__ __forceinline__ void block_argmax(float& u, int& i, float* redu, int* redi) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, nw = (blockDim.x + 63) >> 6;
  wave_argmax(u, i);
  __syncthreads();
  if (l == 0) { redu[w] = u; redi[w] = i; }
  __syncthreads();
  u = redu[0];
  i = redi[0];
  for (int k = 1; k < nw; ++k)
    if (better(redu[k], redi[k], u, i)) { u = redu[k]; i = redi[k]; }
}

// RoPE for pair k: angle = pos / theta^(2k/hd) for the first nrot pairs, 0
// (identity) beyond.  rope_inv gives 1 / wavelength in double (once per pair)
// as step^k, step = theta^(-2/hd) formed on the host in double, by binary
// powering (relative error ~1e-15; a library pow per pair was a long latency
// chain in the kernels that build RoPE tables); rope_cs forms the angle in
// double, reduces it to [-pi, pi] in double (positions reach 32k+, where an
// fp32 angle would be off by ~1e-3 rad) and takes sin / cos of the reduced
// angle in fp32.
__device__ __forceinline__ double rope_inv(int k, double step, int nrot) {
  if (k >= nrot) return 0.0;
  double acc = 1.0, p = step;
#pragma unroll
  for (int b = 0; b < 12; ++b) {  // k < hd / 2 < 4096
    if ((k >> b) & 1) acc *= p;
    p *= p;
  }
  return acc;
}
__device__ __forceinline__ void rope_cs(int64_t pos, double inv, float& c, float& s) {
  const double two_pi = 6.283185307179586;
  const double ang = (double)pos * inv;
  const double red = ang - rint(ang * (1.0 / two_pi)) * two_pi;
  sincosf((float)red, &s, &c);
}
// The same with the hardware sine / cosine (v_sin_f32 / v_cos_f32, absolute
// error near 1e-6 on the reduced angle): a few instructions instead of the
// library sincosf, for tables built on a critical path.
__device__ __forceinline__ void rope_cs_hw(int64_t pos, double inv, float& c, float& s) {
  const double ang = (double)pos * inv * 0.15915494309189535;  // turns
  const float red = (float)(ang - rint(ang));                  // [-1/2, 1/2] turn
  s = __builtin_amdgcn_sinf(red);
  c = __builtin_amdgcn_cosf(red);
}

// Markov walk pruning bound of vocabulary entry v: ||markov_w2[v]|| times
// max_u ||markov_w1[u]|| (aux[v], aux[V]), with a relative margin for the
// fp32 rounding of the dot products it bounds
__device__ __forceinline__ float walk_bound(const float* aux, int64_t v, int V) {
  return aux[v] * aux[V] * (1.f + 1e-5f);
}

// Philox4x64 with 10 rounds (Salmon, Moraes, Dror, Shaw, "Parallel Random
// Numbers: As Easy as 1, 2, 3", SC 2011): four 64-bit words of counter c
// under key (k0, k1)
__device__ __forceinline__ void philox4x64_10(uint64_t c[4], uint64_t k0, uint64_t k1) {
  constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  constexpr uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += W0;
      k1 += W1;
    }
    const uint64_t hi0 = __umul64hi(M0, c[0]), lo0 = M0 * c[0];
    const uint64_t hi1 = __umul64hi(M1, c[2]), lo1 = M1 * c[2];
    const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
}
// The Gumbel noise of vocabulary entry v at block slot `step` of the key
// stream `seed`: g = -log(-log U), U = (top 23 bits + 1/2) / 2^23 (exact in
// float32) of word v mod 4 of Philox4x64-10 at key (seed, 0), counter
// (v / 4, step, 0, 0)
__device__ __forceinline__ float gumbel_noise(uint64_t seed, int step, int v) {
  uint64_t c[4] = {(uint64_t)(v >> 2), (uint64_t)step, 0ull, 0ull};
  philox4x64_10(c, seed, 0ull);
  const int j = v & 3;
  const uint64_t x = j == 0 ? c[0] : (j == 1 ? c[1] : (j == 2 ? c[2] : c[3]));
  const float u = ((float)(uint32_t)(x >> 41) + 0.5f) * 1.1920928955078125e-07f;  // 2^-23
  return -logf(-logf(u));
}

// gelu_pytorch_tanh in fp32
// (the identity 0.5 (1 + tanh u) = 1 / (1 + exp(-2u)), with the hardware
// exponential and reciprocal: relative error ~1e-6, and no cancellation)
__device__ __forceinline__ float gelu_tanh(float x) {
  const float k0 = 0.7978845608028654f;  // sqrt(2/pi)
  const float u = k0 * (x + 0.044715f * x * x * x);
  return x * __builtin_amdgcn_rcpf(1.f + __expf(-2.f * u));
}

// tanh(x) = 1 - 2 / (exp(2x) + 1) with the hardware exponential and
// reciprocal: absolute error ~3e-7 (it saturates to +-1 cleanly)
__device__ __forceinline__ float tanh_fast(float x) {
  return 1.f - 2.f * __builtin_amdgcn_rcpf(__expf(2.f * x) + 1.f);
}

}  // namespace dsp
