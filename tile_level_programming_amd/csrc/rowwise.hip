// rowwise.hip -- row-wise kernels for gfx950 (MI355X), C ABI in rowwise.h:
// the row softmax and the fused RMSNorm + SiLU.
//
// Method.  The TileLang tutorial's row-wise softmax keeps a row in registers
// and takes its maximum and sum with register-level reductions
// (pro.edgex.exchange summary, paragraph on the fused epilogue and the
// row-wise softmax; datastack.it, section "Cosa copre il tutorial"); the
// production RMSNorm + SiLU kernel of the pages' first summary normalises a
// row by its root mean square and applies SiLU in the same kernel.
//
//     softmax:        y_j = exp(x_j - max x) / sum_j exp(x_j - max x)
//     RMSNorm + SiLU: z_j = x_j / sqrt(mean_j x_j^2 + eps) * g_j,  y_j = z_j / (1 + exp(-z_j))
//
// Both read a row once and write it once, so they are bound by HBM.  A row
// is held in registers by a group of TPR threads (16, 32 or 64 lanes of a
// wave for rows up to 2048 elements, several rows per wave for short rows;
// the whole 256-thread work-group beyond), each thread
// holding CPT chunks of 8 elements loaded with 16-byte loads (element loads
// when the row length is not a multiple of 8).  The reductions run within
// the wave by lane exchanges and, for 256-thread groups, across its four
// waves through LDS.  Arithmetic is fp32; outputs are rounded to nearest
// even.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "rowwise.h"

namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kThreads = 256;
constexpr int kMaxC = 32768;  // 16 chunks of 8 per thread of a 256-thread group

template <bool BF16>
__device__ __forceinline__ float lo16(uint32_t w) {
  if constexpr (BF16) return __builtin_bit_cast(float, w << 16);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
template <bool BF16>
__device__ __forceinline__ float hi16(uint32_t w) {
  if constexpr (BF16) return __builtin_bit_cast(float, w & 0xFFFF0000u);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
template <bool BF16>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (BF16) {
    bf16x2 r;
    r[0] = (__bf16)a;
    r[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, r);
  } else {
    f16x2 r;
    r[0] = (_Float16)a;
    r[1] = (_Float16)b;
    return __builtin_bit_cast(uint32_t, r);
  }
}

// element e (0..7) of a chunk
template <bool BF16>
__device__ __forceinline__ float elem(const u32x4& v, int e) {
  return (e & 1) ? hi16<BF16>(v[e >> 1]) : lo16<BF16>(v[e >> 1]);
}

// reductions over the TPR threads of a row group (TPR = 16, 32 or 64:
// lanes of one wave; 256: the work-group, through LDS)
template <int TPR, bool MAX>
__device__ __forceinline__ float group_reduce(float x, float* red) {
#pragma unroll
  for (int o = (TPR < 64 ? TPR : 64) / 2; o >= 1; o >>= 1) {
    const float y = __shfl_xor(x, o, 64);
    x = MAX ? __builtin_elementwise_maximum(x, y) : x + y;
  }
  if constexpr (TPR == 256) {
    const int wave = threadIdx.x >> 6;
    __syncthreads();  // red[] may still be read by an earlier reduction
    if ((threadIdx.x & 63) == 0) red[wave] = x;
    __syncthreads();
    x = MAX ? __builtin_elementwise_maximum(__builtin_elementwise_maximum(red[0], red[1]),
                                            __builtin_elementwise_maximum(red[2], red[3]))
            : (red[0] + red[1]) + (red[2] + red[3]);
  }
  return x;
}

// OP 0: softmax; OP 1: RMSNorm + SiLU.  VEC: rows are whole 16-byte chunks.
template <bool BF16, int OP, int TPR, int CPT, bool VEC>
__global__ __launch_bounds__(kThreads) void rowwise_kernel(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ g,
                                                           uint16_t* __restrict__ y, int R, int C, float eps) {
  __shared__ float red[4];
  constexpr int RPB = kThreads / TPR;
  const int row = blockIdx.x * RPB + threadIdx.x / TPR;
  const int t = threadIdx.x % TPR;
  // every thread of a 256-thread group takes part in the reductions, so a
  // group past the last row still runs them (on no data)
  const bool live = row < R;
  const uint16_t* xr = x + (size_t)(live ? row : 0) * C;
  uint16_t* yr = y + (size_t)(live ? row : 0) * C;

  // load: chunk i of this thread holds elements 8(i TPR + t) .. +7
  u32x4 v[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int e0 = 8 * (i * TPR + t);
    u32x4 w = {0u, 0u, 0u, 0u};
    if (live && e0 < C) {
      if constexpr (VEC) {
        w = *reinterpret_cast<const u32x4*>(xr + e0);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (e0 + e < C) w[e >> 1] |= (uint32_t)xr[e0 + e] << (16 * (e & 1));
      }
    }
    v[i] = w;
  }
  auto valid = [&](int i, int e) __attribute__((always_inline)) { return 8 * (i * TPR + t) + e < C; };

  if constexpr (OP == 0) {
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < CPT; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (valid(i, e)) m = __builtin_elementwise_maximum(m, elem<BF16>(v[i], e));
    m = group_reduce<TPR, true>(m, red);
    // exp(x - m) as exp2((x - m) log2 e), the difference taken first: m
    // log2 e would overflow for a bf16 row whose maximum is above about
    // 2.4e38 and turn the whole row into NaN
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < CPT; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (valid(i, e)) s += __builtin_amdgcn_exp2f((elem<BF16>(v[i], e) - m) * kLog2e);
    s = group_reduce<TPR, false>(s, red);
    const float inv = 1.f / s;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f((elem<BF16>(v[i], e) - m) * kLog2e) * inv;
      u32x4 o;
#pragma unroll
      for (int k = 0; k < 4; ++k) o[k] = pack2<BF16>(p[2 * k], p[2 * k + 1]);
      v[i] = o;
    }
  } else {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < CPT; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float a = elem<BF16>(v[i], e);  // zero past the end
        ss = __builtin_fmaf(a, a, ss);
      }
    ss = group_reduce<TPR, false>(ss, red);
    const float r = 1.f / sqrtf(ss / (float)C + eps);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int e0 = 8 * (i * TPR + t);
      u32x4 gw = {0u, 0u, 0u, 0u};
      if (e0 < C) {
        if constexpr (VEC) {
          gw = *reinterpret_cast<const u32x4*>(g + e0);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (e0 + e < C) gw[e >> 1] |= (uint32_t)g[e0 + e] << (16 * (e & 1));
        }
      }
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float z = elem<BF16>(v[i], e) * r * elem<BF16>(gw, e);
        p[e] = z * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-z * kLog2e));
      }
      u32x4 o;
#pragma unroll
      for (int k = 0; k < 4; ++k) o[k] = pack2<BF16>(p[2 * k], p[2 * k + 1]);
      v[i] = o;
    }
  }

  // store
  if (!live) return;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int e0 = 8 * (i * TPR + t);
    if (e0 >= C) continue;
    if constexpr (VEC) {
      *reinterpret_cast<u32x4*>(yr + e0) = v[i];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (e0 + e < C) yr[e0 + e] = (uint16_t)(v[i][e >> 1] >> (16 * (e & 1)));
    }
  }
}

template <bool BF16, int OP, int TPR, int CPT>
hipError_t launch3(const uint16_t* x, const uint16_t* g, uint16_t* y, int R, int C, float eps, bool vec,
                   hipStream_t s) {
  constexpr int RPB = kThreads / TPR;
  const unsigned blocks = (unsigned)((R + RPB - 1) / RPB);
  if (vec) rowwise_kernel<BF16, OP, TPR, CPT, true><<<blocks, kThreads, 0, s>>>(x, g, y, R, C, eps);
  else rowwise_kernel<BF16, OP, TPR, CPT, false><<<blocks, kThreads, 0, s>>>(x, g, y, R, C, eps);
  return hipGetLastError();
}

// threads per row and chunks per thread from the row length
template <bool BF16, int OP>
hipError_t launch2(const uint16_t* x, const uint16_t* g, uint16_t* y, int R, int C, float eps, bool vec,
                   hipStream_t s) {
  // short rows: a few rows per wave, so that each thread has up to four
  // 16-byte loads in flight
  const int chunks = (C + 7) / 8;
  if (chunks <= 16) return launch3<BF16, OP, 16, 1>(x, g, y, R, C, eps, vec, s);
  if (chunks <= 32) return launch3<BF16, OP, 16, 2>(x, g, y, R, C, eps, vec, s);
  if (chunks <= 64) return launch3<BF16, OP, 16, 4>(x, g, y, R, C, eps, vec, s);
  if (chunks <= 128) return launch3<BF16, OP, 32, 4>(x, g, y, R, C, eps, vec, s);
  if (chunks <= 256) return launch3<BF16, OP, 64, 4>(x, g, y, R, C, eps, vec, s);
  if (chunks <= 512) return launch3<BF16, OP, 256, 2>(x, g, y, R, C, eps, vec, s);
  if (chunks <= 1024) return launch3<BF16, OP, 256, 4>(x, g, y, R, C, eps, vec, s);
  if (chunks <= 2048) return launch3<BF16, OP, 256, 8>(x, g, y, R, C, eps, vec, s);
  return launch3<BF16, OP, 256, 16>(x, g, y, R, C, eps, vec, s);
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t p = (uintptr_t)a, q = (uintptr_t)b;
  return p < q + nb && q < p + na;
}

fa_status check(const void* x, const void* y, int64_t R, int64_t C, int dtype) {
  if (!x || !y) return FA_ERR_INVALID_ARG;
  if (((uintptr_t)x | (uintptr_t)y) & 1u) return FA_ERR_INVALID_ARG;
  if (R < 1 || C < 1) return FA_ERR_INVALID_ARG;
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (C > kMaxC) return FA_ERR_UNSUPPORTED;
  if (R >= ((int64_t)1 << 31)) return FA_ERR_INVALID_ARG;  // (C <= 32768 keeps R*C*2 below 2^47)
  const size_t bytes = (size_t)(R * C) * 2;
  if (overlaps(x, bytes, y, bytes)) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

}  // namespace

extern "C" fa_status row_softmax(const void* x, void* y, int64_t R, int64_t C, int dtype, void* stream) {
  const fa_status st = check(x, y, R, C, dtype);
  if (st != FA_OK) return st;
  const bool vec = (C % 8) == 0 && (((uintptr_t)x | (uintptr_t)y) & 15u) == 0;
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  uint16_t* yp = static_cast<uint16_t*>(y);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t err = dtype == FA_BF16 ? launch2<true, 0>(xp, nullptr, yp, (int)R, (int)C, 0.f, vec, s)
                                          : launch2<false, 0>(xp, nullptr, yp, (int)R, (int)C, 0.f, vec, s);
  return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

extern "C" fa_status rmsnorm_silu(const void* x, const void* g, void* y, int64_t R, int64_t C, float eps, int dtype,
                                  void* stream) {
  fa_status st = check(x, y, R, C, dtype);
  if (st != FA_OK) return st;
  if (!g || ((uintptr_t)g & 1u)) return FA_ERR_INVALID_ARG;
  if (!(eps >= 0.f) || !isfinite(eps)) return FA_ERR_INVALID_ARG;
  if (overlaps(g, (size_t)C * 2, y, (size_t)(R * C) * 2)) return FA_ERR_INVALID_ARG;
  const bool vec = (C % 8) == 0 && (((uintptr_t)x | (uintptr_t)y | (uintptr_t)g) & 15u) == 0;
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  const uint16_t* gp = static_cast<const uint16_t*>(g);
  uint16_t* yp = static_cast<uint16_t*>(y);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t err = dtype == FA_BF16 ? launch2<true, 1>(xp, gp, yp, (int)R, (int)C, eps, vec, s)
                                          : launch2<false, 1>(xp, gp, yp, (int)R, (int)C, eps, vec, s);
  return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}
