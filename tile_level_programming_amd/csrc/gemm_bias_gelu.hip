// gemm_bias_gelu.hip -- GEMM with a fused bias + GELU epilogue for gfx950
// (MI355X), C ABI in gemm.h.
//
// Method: the TileLang tutorial's tiled tensor-core matrix multiplication,
// extended so that the bias addition and the GELU activation are applied to
// the accumulator while it is still in registers, before the output tile is
// written (pro.edgex.exchange summary, paragraph on the fused GEMM epilogue;
// datastack.it, section "Cosa copre il tutorial"; comrad404.com, sections on
// the tiled GEMM and on fusion).  Computed:
//
//     C = gelu(A W^T + bias),   gelu(x) = x * Phi(x) = x/2 * (1 + erf(x/sqrt(2)))
//
// A [M, K], W [N, K] (the weight layout of a linear layer), bias [N] and C
// [M, N], row-major, fp16 or bf16, accumulation in fp32.
//
// CDNA4 mapping.  One work-group of four waves owns a 128 x 128 tile of C;
// each wave a 64 x 64 quarter, as 2 x 2 blocks of v_mfma_f32_32x32x16.  The
// products are formed transposed, C^T = W A^T: the W fragment is the A
// operand and the A fragment the B operand, so a lane owns one row m of C
// and holds 16 of its columns n in runs of 4 consecutive ones (8-byte
// stores in the epilogue).  Both fragments are 16-byte reads of K-contiguous
// rows.
//
//  * K is streamed in 32-wide slabs through a ring of four LDS stages
//    (A and W slab of a stage: 8 KiB each), loaded three slabs ahead with
//    buffer_load_dwordx4 straight into LDS.  Each lane picks the global
//    16-byte chunk that belongs at its LDS slot, which lays a row's four
//    chunks out XOR-swizzled (chunk c of row r at c ^ ((r >> 2) & 3)): the
//    fragment reads of 16 consecutive rows then hit all 64 banks once.
//  * Rows past M or N lie outside the buffer range and read as zeros;
//    chunks past K get an offset outside the range and read as zeros.
//    Slabs past the end are loaded as zeros too, so every wait has a fixed
//    count.
//  * Work-group ids are remapped so that each XCD runs a contiguous range of
//    tiles, ordered in groups of 8 tile rows: the tiles running together
//    share rows of A and W in their XCD's L2.
//  * Epilogue: acc + bias[n], gelu in fp32 (erff), rounded to nearest even.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "gemm.h"

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr uint32_t kBufferWord3 = 0x00020000u;  // raw buffer resource, gfx9 family
constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;   // a buffer offset past any range: reads zeros
constexpr int kWaves = 4;
constexpr int kBM = 128, kBN = 128, kBK = 32;   // work-group tile and K slab
constexpr int kStages = 4;
constexpr int kGroupM = 8;                      // tile rows per ordering group

struct GemmParams {
  const uint16_t* a;
  const uint16_t* w;
  const uint16_t* bias;  // may be null
  uint16_t* c;
  int M, N, K;
  int tiles_m, tiles_n;
};

template <bool BF16>
__device__ __forceinline__ f32x16 mfma_32x32x16(u32x4 a, u32x4 b, f32x16 acc) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
}

template <bool BF16>
__device__ __forceinline__ float to_f32(uint16_t x) {
  if constexpr (BF16) return __builtin_bit_cast(float, (uint32_t)x << 16);
  else return (float)__builtin_bit_cast(_Float16, x);
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

template <bool BF16>
__device__ __forceinline__ uint16_t round1(float a) {
  return (uint16_t)(pack2<BF16>(a, 0.f) & 0xFFFFu);
}

__device__ __forceinline__ float gelu(float x) {
  return 0.5f * x * (1.f + erff(x * 0.70710678118654752f));
}

__device__ __forceinline__ int xcd_remap(int wg, int n) {
  const int xcd = wg & 7, local = wg >> 3;
  const int per = n >> 3, rem = n & 7;
  const int base = xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per;
  return base + local;
}

template <bool BF16>
__global__ __launch_bounds__(256, 2) void gemm_bias_gelu_kernel(GemmParams p) {
  constexpr int SLAB = kBM * kBK * 2;               // bytes of one A (or W) slab
  constexpr int NLD = SLAB / 16 / (64 * kWaves);    // loads per wave per slab and matrix (2)
  __shared__ u32x4 as0[SLAB / 16], as1[SLAB / 16], as2[SLAB / 16], as3[SLAB / 16];
  __shared__ u32x4 ws0[SLAB / 16], ws1[SLAB / 16], ws2[SLAB / 16], ws3[SLAB / 16];
  auto abuf = [&](int s) __attribute__((always_inline)) -> char* {
    return reinterpret_cast<char*>(s == 0 ? as0 : s == 1 ? as1 : s == 2 ? as2 : as3);
  };
  auto wbuf = [&](int s) __attribute__((always_inline)) -> char* {
    return reinterpret_cast<char*>(s == 0 ? ws0 : s == 1 ? ws1 : s == 2 ? ws2 : ws3);
  };

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int wm = wave & 1, wn = wave >> 1;  // this wave's 64 x 64 quarter

  // tile of this work-group: groups of kGroupM tile rows, column-major inside
  const int t = xcd_remap(blockIdx.x, p.tiles_m * p.tiles_n);
  const int per_group = kGroupM * p.tiles_n;
  const int group = t / per_group;
  const int first_m = group * kGroupM;
  const int gsize = min(kGroupM, p.tiles_m - first_m);
  const int tm = first_m + (t - group * per_group) % gsize;
  const int tn = (t - group * per_group) / gsize;
  const int m0 = tm * kBM, n0 = tn * kBN;

  // buffer resources over the work-group's rows of A and W (rows past M or N
  // are outside the range)
  const uint32_t rowb = (uint32_t)p.K * 2u;
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.a + (size_t)m0 * p.K), (short)0, (uint32_t)min(kBM, p.M - m0) * rowb, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.w + (size_t)n0 * p.K), (short)0, (uint32_t)min(kBN, p.N - n0) * rowb, kBufferWord3);

  // load slots: instruction i of this wave fills 1 KiB block i*4 + wave of a
  // slab; lane l writes its bytes 16l..16l+15, that is row (slot / 4),
  // physical chunk slot % 4, holding logical chunk pc ^ ((row >> 2) & 3)
  uint32_t lrow[NLD];
  int lk[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int slot = (i * kWaves + wave) * 64 + lane;
    const int row = slot >> 2, pc = slot & 3;
    const int c = pc ^ ((row >> 2) & 3);
    lrow[i] = (uint32_t)row * rowb;
    lk[i] = c * 8;
  }
  auto issue = [&](int slab, int stage) __attribute__((always_inline)) {
    const int k0 = slab * kBK;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int k = k0 + lk[i];
      const uint32_t off = k < p.K ? lrow[i] + (uint32_t)k * 2u : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(abuf(stage) + (i * kWaves + wave) * 1024), 16, off,
                                               0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int k = k0 + lk[i];
      const uint32_t off = k < p.K ? lrow[i] + (uint32_t)k * 2u : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(wbuf(stage) + (i * kWaves + wave) * 1024), 16, off,
                                               0, 0, 0);
    }
  };

  // fragment reads: block b (32 rows) of the wave's quarter, k-step s (16
  // wide) of the slab; lane l reads row 32b + l%32, logical chunk 2s + l/32
  const int fr = lane & 31, fh = lane >> 5;
  auto frag = [&](const char* base, int row0, int s) __attribute__((always_inline)) -> u32x4 {
    const int r = row0 + fr;
    const int pc = (2 * s + fh) ^ ((r >> 2) & 3);
    return *reinterpret_cast<const u32x4*>(base + r * (kBK * 2) + pc * 16);
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = (p.K + kBK - 1) / kBK;
  issue(0, 0);
  issue(1, 1);
  issue(2, 2);
  for (int j = 0; j < nk; ++j) {
    const int st = j & 3;
    // slab j has landed once at most the two later slabs' loads are in
    // flight; the barrier makes every wave's part of it visible, and tells
    // that every wave has finished reading stage (j+3)%4 (slab j-1, whose
    // fragments were all consumed by the previous step's products)
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(4 * NLD) : "memory");
    issue(j + 3, (j + 3) & 3);
    const char* at = abuf(st);
    const char* wt = wbuf(st);
#pragma unroll
    for (int s = 0; s < kBK / 16; ++s) {
      u32x4 wf[2], af[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        wf[b] = frag(wt, wn * 64 + b * 32, s);
        af[b] = frag(at, wm * 64 + b * 32, s);
      }
#pragma unroll
      for (int bn = 0; bn < 2; ++bn)
#pragma unroll
        for (int bm = 0; bm < 2; ++bm) acc[bn][bm] = mfma_32x32x16<BF16>(wf[bn], af[bm], acc[bn][bm]);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // epilogue: lane holds C[m][n] for m = m0 + 64wm + 32bm + l%32 and
  // n = n0 + 64wn + 32bn + 8g + 4(l/32) + e (accumulator slot 4g + e)
  const bool vec = (p.N & 3) == 0;
#pragma unroll
  for (int bm = 0; bm < 2; ++bm) {
    const int m = m0 + wm * 64 + bm * 32 + fr;
    if (m >= p.M) continue;
    uint16_t* crow = p.c + (size_t)m * p.N;
#pragma unroll
    for (int bn = 0; bn < 2; ++bn)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int nb = n0 + wn * 64 + bn * 32 + 8 * g + 4 * fh;
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int n = nb + e;
          const float bv = (p.bias && n < p.N) ? to_f32<BF16>(p.bias[n]) : 0.f;
          y[e] = gelu(acc[bn][bm][4 * g + e] + bv);
        }
        if (vec && nb + 3 < p.N) {
          u32x2 v;
          v[0] = pack2<BF16>(y[0], y[1]);
          v[1] = pack2<BF16>(y[2], y[3]);
          *reinterpret_cast<u32x2*>(crow + nb) = v;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (nb + e < p.N) crow[nb + e] = round1<BF16>(y[e]);
        }
      }
  }
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

}  // namespace

extern "C" fa_status gemm_bias_gelu(const void* a, const void* w, const void* bias, void* c, int64_t M, int64_t N,
                                    int64_t K, int dtype, void* stream) {
  if (!a || !w || !c) return FA_ERR_INVALID_ARG;
  if (((uintptr_t)a | (uintptr_t)w | (uintptr_t)c) & 15u) return FA_ERR_INVALID_ARG;
  if (bias && ((uintptr_t)bias & 1u)) return FA_ERR_INVALID_ARG;
  if (M < 1 || N < 1 || K < 1) return FA_ERR_INVALID_ARG;
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (K % 8 != 0) return FA_ERR_UNSUPPORTED;
  const int64_t lim = (int64_t)1 << 31;
  if (M >= lim || N >= lim || K >= lim) return FA_ERR_INVALID_ARG;
  // a work-group's buffer range, 128 rows of 2K bytes, and the tile count
  // stay inside 32 bits
  if ((int64_t)kBM * K * 2 >= (int64_t)kOutOfRange) return FA_ERR_INVALID_ARG;
  const int64_t tiles_m = (M + kBM - 1) / kBM, tiles_n = (N + kBN - 1) / kBN;
  if (tiles_m * tiles_n >= lim) return FA_ERR_INVALID_ARG;
  const size_t a_bytes = (size_t)M * (size_t)K * 2, w_bytes = (size_t)N * (size_t)K * 2;
  const size_t c_bytes = (size_t)M * (size_t)N * 2, b_bytes = (size_t)N * 2;
  if (overlaps(c, c_bytes, a, a_bytes) || overlaps(c, c_bytes, w, w_bytes) ||
      (bias && overlaps(c, c_bytes, bias, b_bytes)))
    return FA_ERR_INVALID_ARG;

  GemmParams p;
  p.a = static_cast<const uint16_t*>(a);
  p.w = static_cast<const uint16_t*>(w);
  p.bias = static_cast<const uint16_t*>(bias);
  p.c = static_cast<uint16_t*>(c);
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.tiles_m = (int)tiles_m;
  p.tiles_n = (int)tiles_n;
  void* args[] = {&p};
  const void* fn = dtype == FA_BF16 ? reinterpret_cast<const void*>(&gemm_bias_gelu_kernel<true>)
                                    : reinterpret_cast<const void*>(&gemm_bias_gelu_kernel<false>);
  const hipError_t err = hipLaunchKernel(fn, dim3((unsigned)(tiles_m * tiles_n)), dim3(64 * kWaves), args, 0,
                                         static_cast<hipStream_t>(stream));
  return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}
