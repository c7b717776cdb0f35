// On-device quantizers: FP32 data -> element codes + block scales, the step
// that feeds the GEMM operands.
//
// MX ("PyTorch on AMD GPUs gains a FlyDSL backend", Interpretation): one E8M0
// power-of-two scale per 32 consecutive values along K.  The exponent is
// X = floor(log2(amax / fmt_max)) taken exactly (X = -127 for an all-zero
// block, clamped to [-127, 127]); elements are x * 2^-X (exact in FP32)
// rounded to the nearest code, ties to the even code, saturating at
// +-fmt_max.
//
// Groupwise ("Add FlyDSL grouped groupwise FP8 GEMM for ROCm", PR body and
// commit messages): E4M3 with one FP32 scale per row and 128-value K block,
// s = amax / 448 (an FP32 quotient, 1.0 for an all-zero block), elements the
// FP32 quotient x / s rounded to the nearest E4M3 code; the scales are
// written in the per-group block layout the grouped GEMM reads: (row r of
// group g, k block kb) at start_g * (K/128) + (r - start_g) + kb * M_g.
//
// The weights ("Add FlyDSL grouped groupwise FP8 GEMM for ROCm", PR body:
// 128x128 weight blocks) follow the activations' rule per 128 x 128 block,
// scales [G, N/128, K/128] row-major.
//
// Tensor-wise ("Experimental FlyDSL GEMM backend for TE PyTorch", Supported
// Data Types: tensor-wise FP8): one FP32 dequant scale for the whole tensor
// from its own amax, s = amax / fmt_max as an FP32 quotient (1.0 for an
// all-zero tensor), elements the FP32 quotient x / s rounded to the nearest
// E4M3 or E5M2 code: the groupwise rule with the tensor as one block.
//
// All are HBM-bound streams: 4 bytes read per element, 1 (FP8) or 1/2
// (FP4) written, plus the scales (the tensor-wise quantizer reads the data
// twice: once for the amax, once to encode).
#pragma once
#include "common.hpp"

namespace mxg {

// Nearest code of y (FP32, finite) in format FMT, ties to the even code,
// saturating; the sign bit is kept (a negative value that rounds to zero
// gives the negative-zero code).  The quotient a * 2^(MB - E) of a normal
// magnitude a with exponent E is exact and lies in [2^MB, 2^(MB+1)); its
// round-to-nearest-even integer is the mantissa with the implicit bit, and a
// carry to 2^(MB+1) moves to the next exponent through the plain addition.
template <int FMT>
__device__ inline uint32_t encode_nearest(float y) {
  constexpr int MB = FMT == F_E4M3 ? 3 : (FMT == F_E5M2 ? 2 : 1);         // mantissa bits
  constexpr int BIAS = FMT == F_E4M3 ? 7 : (FMT == F_E5M2 ? 15 : 1);
  constexpr uint32_t TOP = FMT == F_E4M3 ? 0x7Eu : (FMT == F_E5M2 ? 0x7Bu : 0x7u);
  constexpr float FMAX = FMT == F_E4M3 ? 448.0f : (FMT == F_E5M2 ? 57344.0f : 6.0f);
  constexpr int EMIN = 1 - BIAS;                                            // smallest normal exponent
  const uint32_t neg = __float_as_uint(y) >> 31;
  const float a = fabsf(y);
  uint32_t c;
  if (a >= FMAX) {
    c = TOP;
  } else if (a < ldexpf(1.0f, EMIN)) {
    // subnormal codes m * 2^(EMIN - MB); m = 2^MB is the smallest normal
    c = (uint32_t)rintf(ldexpf(a, MB - EMIN));
  } else {
    const int E = ilogbf(a);
    const uint32_t q = (uint32_t)rintf(ldexpf(a, MB - E));
    c = ((uint32_t)(E + BIAS) << MB) + (q - (1u << MB));
    if (c > TOP) c = TOP;
  }
  return c | (neg << (FMT == F_E2M1 ? 3 : 7));
}

// Four E4M3 (E5M2) codes of a, b, c, d (finite) by gfx950's conversion
// instruction (round to nearest even, OCP formats), after saturating to
// +-448 (+-57344) so that no value overflows: the same decision as
// encode_nearest, in one instruction per pair.  encode_nearest stays the
// definition the tests compare both against (and the E2M1 encoder).
__device__ inline uint32_t encode4_e4m3_hw(float a, float b, float c, float d) {
  auto sat = [](float v) { return fminf(fmaxf(v, -448.0f), 448.0f); };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(a), sat(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(c), sat(d), w, true);
  return (uint32_t)w;
}

__device__ inline uint32_t encode4_e5m2_hw(float a, float b, float c, float d) {
  auto sat = [](float v) { return fminf(fmaxf(v, -57344.0f), 57344.0f); };
  int w = __builtin_amdgcn_cvt_pk_bf8_f32(sat(a), sat(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_bf8_f32(sat(c), sat(d), w, true);
  return (uint32_t)w;
}

// X = floor(log2(amax / fmt_max)), exactly: with amax = f 2^e (f in
// [0.5, 1)) and fmt_max = g 2^h (g in [0.5, 1)), the ratio is (f/g) 2^(e-h)
// with f/g in (0.5, 2), so X = e - h, less one when f < g.
template <int FMT>
__device__ inline int e8m0_exponent(float amax) {
  if (!(amax > 0.0f)) return -127;
  constexpr float G = FMT == F_E2M1 ? 0.75f : 0.875f;                      // 6 = 0.75 2^3; 448 = 0.875 2^9
  constexpr int H = FMT == F_E4M3 ? 9 : (FMT == F_E5M2 ? 16 : 3);           // 57344 = 0.875 2^16
  int e;
  const float f = frexpf(amax, &e);
  int X = e - H - (f < G ? 1 : 0);
  return X < -127 ? -127 : (X > 127 ? 127 : X);
}

__device__ inline float max4(float a, float b, float c, float d) { return fmaxf(fmaxf(a, b), fmaxf(c, d)); }

// One thread per 8 consecutive values (two 16-byte loads); the four threads
// of a 32-value block are consecutive lanes and exchange their partial
// maxima by shuffles.  rows * K % 32 == 0, so a block's four lanes are in or
// out of range together.
template <int FMT>
__global__ __launch_bounds__(256) void quant_mx_kernel(const float *__restrict__ x, uint8_t *__restrict__ codes,
                                                       uint8_t *__restrict__ scales, int64_t n8) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n8) return;
  const float4 u = ((const float4 *)x)[2 * t];
  const float4 v = ((const float4 *)x)[2 * t + 1];
  float m = fmaxf(max4(fabsf(u.x), fabsf(u.y), fabsf(u.z), fabsf(u.w)),
                  max4(fabsf(v.x), fabsf(v.y), fabsf(v.z), fabsf(v.w)));
  m = fmaxf(m, __shfl_xor(m, 1, 4));
  m = fmaxf(m, __shfl_xor(m, 2, 4));
  const int X = e8m0_exponent<FMT>(m);
  const float inv = ldexpf(1.0f, -X);
  const float y[8] = {u.x * inv, u.y * inv, u.z * inv, u.w * inv, v.x * inv, v.y * inv, v.z * inv, v.w * inv};
  if constexpr (FMT == F_E2M1) {
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) w |= encode_nearest<FMT>(y[j]) << (4 * j);
    ((uint32_t *)codes)[t] = w;
  } else if constexpr (FMT == F_E4M3) {
    ((uint2 *)codes)[t] = make_uint2(encode4_e4m3_hw(y[0], y[1], y[2], y[3]), encode4_e4m3_hw(y[4], y[5], y[6], y[7]));
  } else {
    ((uint2 *)codes)[t] = make_uint2(encode4_e5m2_hw(y[0], y[1], y[2], y[3]), encode4_e5m2_hw(y[4], y[5], y[6], y[7]));
  }
  if ((t & 3) == 0) scales[t >> 2] = (uint8_t)(X + 127);
}

// Groupwise activations.  Each workgroup first builds the clamped prefix
// sums of m_sizes in LDS (pre[g] = min(sum of max(m_h, 0) over h < g, totM),
// g = 0..G, by one wave: each lane sums a run of groups, then a 64-lane
// inclusive scan); rows at or past pre[G] belong to no group and are not
// written.  Then it walks 1 x 128 blocks, 16 per pass (16 lanes per block,
// 8 values each), finding a row's group by binary search over pre.
constexpr int QG_MAX = 1024;

__global__ __launch_bounds__(256) void quant_group_act_kernel(const int64_t *__restrict__ m_sizes, int G,
                                                              const float *__restrict__ x,
                                                              uint8_t *__restrict__ codes, float *__restrict__ xs,
                                                              int64_t totM, int64_t K) {
  __shared__ int pre[QG_MAX + 1];
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int per = (G + 63) / 64;
    const int g0 = lane * per;
    int64_t run = 0;
    for (int j = 0; j < per; ++j) {
      const int g = g0 + j;
      if (g < G) {
        const int64_t s = m_sizes[g];
        run += s > 0 ? s : 0;
      }
    }
    // inclusive scan of the lanes' run sums
    int64_t inc = run;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int64_t o = __shfl_up(inc, d, 64);
      if (lane >= d) inc += o;
    }
    int64_t acc = inc - run;                    // exclusive prefix at g0
    for (int j = 0; j < per; ++j) {
      const int g = g0 + j;
      if (g <= G) pre[g] = (int)(acc < totM ? acc : totM);
      if (g < G) {
        const int64_t s = m_sizes[g];
        acc += s > 0 ? s : 0;
      }
    }
    if (lane == 63 && g0 + per <= G) pre[G] = (int)(acc < totM ? acc : totM);
  }
  __syncthreads();
  const int covered = pre[G];
  // block counts stay below 2^29 (the entry point bounds totM * K/128), so
  // the row of a block comes from a 32-bit division
  const uint32_t nkb = (uint32_t)(K / 128);
  const uint32_t nblk = (uint32_t)covered * nkb;
  const int sub = threadIdx.x & 15;
  for (uint32_t b = blockIdx.x * 16u + (threadIdx.x >> 4); b < nblk; b += gridDim.x * 16u) {
    const int r = (int)(b / nkb);
    const int64_t kb = (int64_t)(b - (uint32_t)r * nkb);
    // group of row r: the last g with pre[g] <= r (pre[g+1] > r then)
    int lo = 0, hi = G;                          // pre[lo] <= r < pre[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (pre[mid] <= r) lo = mid; else hi = mid;
    }
    const int start = pre[lo], mg = pre[lo + 1] - pre[lo];
    const float4 *src = (const float4 *)(x + (int64_t)r * K + 128 * kb + 8 * sub);
    const float4 u = src[0], v = src[1];
    float m = fmaxf(max4(fabsf(u.x), fabsf(u.y), fabsf(u.z), fabsf(u.w)),
                    max4(fabsf(v.x), fabsf(v.y), fabsf(v.z), fabsf(v.w)));
    m = fmaxf(m, __shfl_xor(m, 1, 16));
    m = fmaxf(m, __shfl_xor(m, 2, 16));
    m = fmaxf(m, __shfl_xor(m, 4, 16));
    m = fmaxf(m, __shfl_xor(m, 8, 16));
    const float s = m > 0.0f ? __fdiv_rn(m, 448.0f) : 1.0f;
    const float q[8] = {__fdiv_rn(u.x, s), __fdiv_rn(u.y, s), __fdiv_rn(u.z, s), __fdiv_rn(u.w, s),
                        __fdiv_rn(v.x, s), __fdiv_rn(v.y, s), __fdiv_rn(v.z, s), __fdiv_rn(v.w, s)};
    const uint32_t lo4 = encode4_e4m3_hw(q[0], q[1], q[2], q[3]);
    const uint32_t hi4 = encode4_e4m3_hw(q[4], q[5], q[6], q[7]);
    *(uint2 *)(codes + (int64_t)r * K + 128 * kb + 8 * sub) = make_uint2(lo4, hi4);
    if (sub == 0) xs[(int64_t)start * nkb + (r - start) + kb * mg] = s;
  }
}

// Groupwise weights: one workgroup per 128 x 128 block of w [G, N, K] (K
// contiguous).  Thread t reads float4 chunk t % 32 of rows 2i + (t / 32) % 2
// of its wave's 32-row band (i = 0..15), so each load instruction covers two
// whole 512-byte rows; the block maximum goes through the wave (shuffles) and
// LDS (four waves).
__global__ __launch_bounds__(256) void quant_group_weight_kernel(const float *__restrict__ w,
                                                                 uint8_t *__restrict__ codes,
                                                                 float *__restrict__ ws, int64_t N, int64_t K) {
  __shared__ float wmax[4];
  const int64_t nb = N / 128, kb = K / 128;
  const int64_t blk = blockIdx.x;
  const int64_t g = blk / (nb * kb), bn = (blk / kb) % nb, bk = blk % kb;
  const int64_t origin = (g * N + bn * 128) * K + bk * 128;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int chunk = lane & 31, half = lane >> 5;
  float4 v[16];
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t row = wave * 32 + 2 * i + half;
    v[i] = *(const float4 *)(w + origin + row * K + 4 * chunk);
    m = fmaxf(m, max4(fabsf(v[i].x), fabsf(v[i].y), fabsf(v[i].z), fabsf(v[i].w)));
  }
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
  if (lane == 0) wmax[wave] = m;
  __syncthreads();
  m = max4(wmax[0], wmax[1], wmax[2], wmax[3]);
  const float s = m > 0.0f ? __fdiv_rn(m, 448.0f) : 1.0f;
  if (threadIdx.x == 0) ws[blk] = s;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t row = wave * 32 + 2 * i + half;
    const uint32_t c = encode4_e4m3_hw(__fdiv_rn(v[i].x, s), __fdiv_rn(v[i].y, s), __fdiv_rn(v[i].z, s),
                                       __fdiv_rn(v[i].w, s));
    *(uint32_t *)(codes + origin + row * K + 4 * chunk) = c;
  }
}

// Tensor-wise quantizer, four launches on one stream and no scratch: the
// caller's scale word holds the amax (as FP32 bits, which order like
// unsigned integers for non-negative values) until the last launch turns it
// into the scale.
__global__ void tensor_amax_clear_kernel(uint32_t *amax_bits) {
  if (threadIdx.x == 0) amax_bits[threadIdx.x] = 0u;
}

// Grid-stride over groups of 8 values, four groups (eight 16-byte loads)
// in flight per thread; block maximum by wave shuffles and LDS, then one
// atomic maximum per block.
__global__ __launch_bounds__(256) void tensor_amax_kernel(const float *__restrict__ x, int64_t n8,
                                                          uint32_t *amax_bits) {
  __shared__ float wmax[4];
  const float4 *x4 = (const float4 *)x;
  auto absmax = [](const float4 &u) { return max4(fabsf(u.x), fabsf(u.y), fabsf(u.z), fabsf(u.w)); };
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  float m = 0.0f;
  for (; t + 3 * stride < n8; t += 4 * stride) {
    float4 u[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u[2 * j] = x4[2 * (t + j * stride)];
      u[2 * j + 1] = x4[2 * (t + j * stride) + 1];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, absmax(u[j]));
  }
  for (; t < n8; t += stride) m = fmaxf(m, fmaxf(absmax(x4[2 * t]), absmax(x4[2 * t + 1])));
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) wmax[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0) atomicMax(amax_bits, __float_as_uint(max4(wmax[0], wmax[1], wmax[2], wmax[3])));
}

template <int FMT>
__device__ inline float tensor_scale(uint32_t amax_bits) {
  constexpr float FMAX = FMT == F_E4M3 ? 448.0f : 57344.0f;
  const float amax = __uint_as_float(amax_bits);
  return amax > 0.0f ? __fdiv_rn(amax, FMAX) : 1.0f;
}

// One thread per 8 consecutive values.
template <int FMT>
__global__ __launch_bounds__(256) void tensor_quant_kernel(const float *__restrict__ x, uint8_t *__restrict__ codes,
                                                           const uint32_t *__restrict__ amax_bits, int64_t n8) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n8) return;
  const float s = tensor_scale<FMT>(*amax_bits);
  const float4 u = ((const float4 *)x)[2 * t];
  const float4 v = ((const float4 *)x)[2 * t + 1];
  const float y[8] = {__fdiv_rn(u.x, s), __fdiv_rn(u.y, s), __fdiv_rn(u.z, s), __fdiv_rn(u.w, s),
                      __fdiv_rn(v.x, s), __fdiv_rn(v.y, s), __fdiv_rn(v.z, s), __fdiv_rn(v.w, s)};
  if constexpr (FMT == F_E4M3)
    ((uint2 *)codes)[t] = make_uint2(encode4_e4m3_hw(y[0], y[1], y[2], y[3]), encode4_e4m3_hw(y[4], y[5], y[6], y[7]));
  else
    ((uint2 *)codes)[t] = make_uint2(encode4_e5m2_hw(y[0], y[1], y[2], y[3]), encode4_e5m2_hw(y[4], y[5], y[6], y[7]));
}

// The amax in the scale word becomes the scale (after every encoder thread
// has read the amax: the launch follows the encoder on the stream).
template <int FMT>
__global__ void tensor_scale_kernel(uint32_t *scale_word) {
  if (threadIdx.x == 0) scale_word[threadIdx.x] = __float_as_uint(tensor_scale<FMT>(scale_word[threadIdx.x]));
}

}  // namespace mxg
