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
// CDNA4 mapping.  One work-group of four waves (one per SIMD) owns a
// 256 x 256 tile of C; the waves form a 2 (n) x 2 (m) grid, each owning 128
// columns n by 128 rows m as 4 x 4 blocks of v_mfma_f32_32x32x16 (256
// accumulator registers).  The products are formed transposed, C^T = W A^T:
// the W fragment is the A operand and the A fragment the B operand, so a
// lane owns one row m of C and holds 16 of its columns n per block in runs
// of 4 consecutive ones (8-byte stores in the epilogue).  Both fragments are
// 16-byte reads of K-contiguous rows.
//
//  * K is streamed in 64-wide slabs with buffer_load_dwordx4 straight into
//    LDS: A through two stages, W through three (32 KiB per slab and
//    matrix, 160 KiB in all).  A slab row is one 128-byte line of A or W, so
//    every load instruction fetches whole lines.  Each lane picks the global
//    16-byte chunk that belongs at its LDS slot, which lays a row's eight
//    chunks out XOR-swizzled (chunk c of row r at c ^ ((r >> 1) & 7)): the
//    fragment reads of 16 consecutive rows then hit all 64 banks once.
//  * A step computes one slab in four k-steps of 16, reading each k-step's
//    fragments during the previous one's products.  Halfway through the last
//    k-step every wave waits for the next slab's loads and meets the others
//    at a barrier; the remaining products then cover the first fragment
//    reads of the next slab.  The loads are spread over the products so
//    that the address unit is never flooded: A slab j+2 goes into the stage
//    A slab j leaves at that barrier, two loads right after it and the rest
//    during the next step's first k-step; W slab j+2 goes into the third W
//    stage during the middle k-steps of step j, a whole step before it is
//    needed.
//  * Rows past M or N lie outside the buffer range and read as zeros;
//    slabs past the end go through a resource with an empty range; when K
//    is not a multiple of 64, chunks past K get an offset outside the range
//    (both read as zeros and touch no memory).
//  * Work-group ids are remapped so that each XCD runs a contiguous range of
//    tiles, ordered in groups of 4 tile rows (column-major inside a group):
//    the 32 tiles an XCD runs together are 4 rows by 8 columns of tiles, and
//    share rows of A and W in its L2.
//  * Epilogue: acc + bias[n] (read after the K loop), gelu in fp32 with the
//    Abramowitz-Stegun erf approximation, rounded to nearest even, staged
//    through the (then idle) LDS stages so that C is written in whole
//    cache lines.

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
constexpr int kGroupM = 4;                      // tile rows per ordering group
// scheduling-group masks of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedMfma = 0x008;
constexpr int kSchedVmem = 0x010;
constexpr int kSchedDsRead = 0x100;

// Tile configuration: four waves in a 2 (n) x 2 (m) grid, each owning
// 4 x 4 blocks of 32 x 32 of a 256 x 256 tile; K in 64-wide slabs, two LDS
// stages for A and three for W.
constexpr int kWaves = 4;
constexpr int WT = 128;                    // wave-tile edge
constexpr int NB = WT / 32;                // 32 x 32 blocks per wave-tile edge
constexpr int BM = 256, BN = 256;          // tile of C per work-group
constexpr int BK = 64;                     // slab width: one 128-byte line per row
constexpr int ROWB = BK * 2;               // bytes of a slab row
constexpr int CPR = BK / 8;                // 16-byte chunks per slab row
constexpr int SLAB = 256 * ROWB;           // bytes of one matrix's slab
constexpr int NLA = SLAB / (16 * 64 * kWaves);  // loads per wave and matrix per slab
constexpr int NL = 2 * NLA;                // loads per wave per slab (A first, then W)
constexpr int KS = BK / 16;                // k-steps per slab
static_assert(NLA * 16 * 64 * kWaves == SLAB, "slabs split over the waves");
static_assert(KS == 4, "the step is written for four k-steps");

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

// gelu(x) = x * Phi(x).  Phi from the erf approximation 7.1.26 of
// Abramowitz and Stegun (|error of erf| <= 1.5e-7 for all x), applied to
// |x|/sqrt(2):  h = 1 - Phi(|x|) = (a1 t + a2 t^2 + ... + a5 t^5) e^(-x^2/2) / 2
// with t = 1 / (1 + p |x|/sqrt(2)); Phi(x) = 1 - h for x >= 0 and h for
// x < 0 (no cancellation in the negative tail).  About a dozen instructions
// and no branch; the error (<= 7.5e-8 |x|) is far below the output rounding.
__device__ __forceinline__ float gelu(float x) {
  const float z = fabsf(x) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.3275911f, z, 1.f));
  float poly = __builtin_fmaf(1.061405429f, t, -1.453152027f);
  poly = __builtin_fmaf(poly, t, 1.421413741f);
  poly = __builtin_fmaf(poly, t, -0.284496736f);
  poly = __builtin_fmaf(poly, t, 0.254829592f);
  poly *= t;
  const float e = __builtin_amdgcn_exp2f(-z * z * 1.4426950408889634f);  // e^(-z^2)
  const float h = 0.5f * poly * e;
  return x * (x >= 0.f ? 1.f - h : h);
}

template <int I>
struct Int { static constexpr int value = I; };

// f(Int<I>) for I = B .. E-1, unrolled at compile time
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(Int<B>{});
    static_for<B + 1, E>(f);
  }
}

__device__ __forceinline__ int xcd_remap(int wg, int n) {
  const int xcd = wg & 7, local = wg >> 3;
  const int per = n >> 3, rem = n & 7;
  const int base = xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per;
  return base + local;
}

// KTAIL: K is not a multiple of BK, and the last slab's chunks past K must
// read as zeros lane by lane
template <bool BF16, bool KTAIL>
__global__ __launch_bounds__(64 * kWaves, 1) void gemm_bias_gelu_kernel(GemmParams p) {
  // one array per stage and matrix: the compiler can then tell that the
  // loads streaming into one stage never alias the reads from another
  __shared__ u32x4 as0[SLAB / 16], as1[SLAB / 16], ws0[SLAB / 16], ws1[SLAB / 16], ws2[SLAB / 16];
  auto abuf = [&](int s) __attribute__((always_inline)) -> char* { return reinterpret_cast<char*>(s == 0 ? as0 : as1); };
  auto wbuf = [&](int s) __attribute__((always_inline)) -> char* { return reinterpret_cast<char*>(s == 0 ? ws0 : s == 1 ? ws1 : ws2); };
  // chunk c of slab row r sits at physical chunk c ^ swz(r): the 16-byte
  // fragment reads of 16 consecutive rows then cover all 64 banks once
  auto swz = [](int r) __attribute__((always_inline)) { return (r >> 1) & (CPR - 1); };

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int wm = wave & 1, wn = wave >> 1;  // this wave's part of the tile

  // tile of this work-group: groups of kGroupM tile rows, column-major inside
  const int t = xcd_remap(blockIdx.x, p.tiles_m * p.tiles_n);
  const int per_group = kGroupM * p.tiles_n;
  const int group = t / per_group;
  const int first_m = group * kGroupM;
  const int gsize = min(kGroupM, p.tiles_m - first_m);
  const int tm = first_m + (t - group * per_group) % gsize;
  const int tn = (t - group * per_group) / gsize;
  const int m0 = tm * BM, n0 = tn * BN;

  // buffer resources over the work-group's rows of A and W (rows past M or N
  // are outside the range)
  const uint32_t rowg = (uint32_t)p.K * 2u;
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.a + (size_t)m0 * p.K), (short)0, (uint32_t)min(BM, p.M - m0) * rowg, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.w + (size_t)n0 * p.K), (short)0, (uint32_t)min(BN, p.N - n0) * rowg, kBufferWord3);

  // load slots: load i of a matrix fills 1 KiB block i * kWaves + wave of
  // its slab; lane l writes bytes 16l .. 16l + 15 of it, that is row
  // 32i + 8 wave + l/8, physical chunk l % 8, which holds logical chunk
  // (l % 8) ^ swz(row) = (l % 8) ^ (4 (wave & 1) + l / 16): the same chunk
  // for every i (32i + 8 wave moves swz by a multiple of 8 rows), so one
  // offset per lane serves every load of A and W.
  static_assert(kWaves == 4 && CPR == 8, "the slot formula assumes four waves and 8 chunks per row");
  const int lk = ((lane & 7) ^ ((wave & 1) * 4 + (lane >> 4))) * 8;  // the lane's k within a slab
  const uint32_t lbase = (uint32_t)(wave * 8 + (lane >> 3)) * rowg + (uint32_t)lk * 2u;
  // A slab past the end (the last steps load two) goes through a resource
  // with an empty range: its loads read zeros and touch no memory.  With
  // K a multiple of BK that uniform choice is the only check; otherwise
  // each lane also checks its chunk against K.
  const __amdgpu_buffer_rsrc_t rnone = __builtin_amdgcn_make_buffer_rsrc((void*)p.a, (short)0, 0u, kBufferWord3);
  auto issue = [&](int slab, int stage, auto i0_tag, auto i1_tag, int wstage = -1) __attribute__((always_inline)) {
    constexpr int I0 = decltype(i0_tag)::value, I1 = decltype(i1_tag)::value;
    const int k0 = slab * BK;
    const bool live = k0 < p.K;
    const __amdgpu_buffer_rsrc_t rA = live ? ra : rnone, rW = live ? rw : rnone;
    const bool lane_in = !KTAIL || k0 + lk < p.K;
    static_for<I0, I1>([&](auto it) {
      constexpr int q = decltype(it)::value;
      constexpr int i = q % NLA;
      uint32_t off = lbase + ((uint32_t)(i * 32) * rowg + (uint32_t)k0 * 2u);
      if constexpr (KTAIL) off = lane_in ? off : kOutOfRange;
      if constexpr (q < NLA)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_void*)(abuf(stage) + (i * kWaves + wave) * 1024), 16, off,
                                                 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rW, (lds_void*)(wbuf(wstage < 0 ? stage : wstage) + (i * kWaves + wave) * 1024),
                                                 16, off, 0, 0, 0);
    });
  };

  // fragment of block row0.. (32 rows), k-step s (16 wide) of a slab: lane l
  // reads row row0 + l%32, logical chunk 2s + l/32
  const int fr = lane & 31, fh = lane >> 5;
  auto frag = [&](const char* base, int row0, int s) __attribute__((always_inline)) -> u32x4 {
    const int r = row0 + fr;
    const int pc = (2 * s + fh) ^ swz(r);
    return *reinterpret_cast<const u32x4*>(base + r * ROWB + pc * 16);
  };
  // the fragments of k-step s, in the order the products use them
  auto read = [&](u32x4* wf, u32x4* af, const char* wt, const char* at, int s) __attribute__((always_inline)) {
    wf[0] = frag(wt, wn * WT, s);
#pragma unroll
    for (int b = 0; b < NB; ++b) af[b] = frag(at, wm * WT + b * 32, s);
#pragma unroll
    for (int b = 1; b < NB; ++b) wf[b] = frag(wt, wn * WT + b * 32, s);
  };

  f32x16 acc[NB][NB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  // products of block rows bn0 .. bn1-1 with one k-step's fragments
  auto mm = [&](const u32x4* wf, const u32x4* af, int bn0, int bn1) __attribute__((always_inline)) {
#pragma unroll
    for (int bn = bn0; bn < bn1; ++bn)
#pragma unroll
      for (int bm = 0; bm < NB; ++bm) acc[bn][bm] = mfma_32x32x16<BF16>(wf[bn], af[bm], acc[bn][bm]);
  };

  constexpr int NF = 2 * NB;   // fragment reads per k-step
  constexpr int NM = NB * NB;  // products per k-step
  constexpr int NP = NM / 2;   // products of the last k-step after the barrier
  constexpr int NLA1 = 2;      // A loads of a slab issued after the barrier two steps ahead
  // the order of one k-step: a fragment read after every other product,
  // NR loads spread evenly over the products
  auto kstep_order = [&](auto nr_tag) __attribute__((always_inline)) {
    constexpr int NR = decltype(nr_tag)::value;
    static_for<0, NM>([&](auto it) {
      constexpr int i = decltype(it)::value;
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      if constexpr (i % 2 == 1 && i / 2 < NF) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      if constexpr (i * NR / NM != (i + 1) * NR / NM) __builtin_amdgcn_sched_group_barrier(kSchedVmem, 1, 0);
    });
  };
  u32x4 w0[NB], a0[NB], w1[NB], a1[NB];

  // step j: A slab j in stage SA = j % 2, W slab j in stage SW = j % 3
  // (passed at compile time).  On entry the k-step-0 fragments of slab j
  // are in w0/a0, and W slab j+1 and the first NLA1 loads of A slab j+1 are
  // in flight, in that order.
  auto step = [&](int j, auto sa_tag, auto sw_tag) __attribute__((always_inline)) {
    constexpr int SA = decltype(sa_tag)::value, SW = decltype(sw_tag)::value;
    constexpr int SW2 = (SW + 2) % 3;  // W stage of slab j-1, read by every wave before the last barrier
    const char* at = abuf(SA);
    const char* wt = wbuf(SW);
    // k-step 0, with the rest of A slab j+1's loads
    issue(j + 1, SA ^ 1, Int<NLA1>{}, Int<NLA>{});
    read(w1, a1, wt, at, 1);
    mm(w0, a0, 0, NB);
    kstep_order(Int<NLA - NLA1>{});
    // k-steps 1 and 2, with W slab j+2's loads (after every A load of slab
    // j+1, so that the wait below can leave them in flight)
    read(w0, a0, wt, at, 2);
    issue(j + 2, 0, Int<NLA>{}, Int<NLA + NLA / 2>{}, SW2);
    mm(w1, a1, 0, NB);
    kstep_order(Int<NLA / 2>{});
    read(w1, a1, wt, at, 3);
    issue(j + 2, 0, Int<NLA + NLA / 2>{}, Int<NL>{}, SW2);
    mm(w0, a0, 0, NB);
    kstep_order(Int<NLA - NLA / 2>{});
    // k-step 3: half of the products, then the wait for slab j+1 (only W
    // slab j+2's loads, the last issued, stay in flight) and the barrier
    // after which every wave has read all of A slab j: its stage takes the
    // first loads of A slab j+2 while the rest of the products cover the
    // reads of slab j+1's first fragments
    mm(w1, a1, 0, NB / 2);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(NLA) : "memory");
    __builtin_amdgcn_sched_barrier(0);
    read(w0, a0, wbuf((SW + 1) % 3), abuf(SA ^ 1), 0);
    issue(j + 2, SA, Int<0>{}, Int<NLA1>{});
    mm(w1, a1, NB / 2, NB);
    static_for<0, NP>([&](auto it) {
      constexpr int i = decltype(it)::value;
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      if constexpr (i * NF / NP != (i + 1) * NF / NP)
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, (i + 1) * NF / NP - i * NF / NP, 0);
      if constexpr (i * NLA1 / NP != (i + 1) * NLA1 / NP)
        __builtin_amdgcn_sched_group_barrier(kSchedVmem, (i + 1) * NLA1 / NP - i * NLA1 / NP, 0);
    });
  };

  const int nk = (p.K + BK - 1) / BK;
  // prologue: slab 0, then W slab 1, then A slab 1's first loads
  issue(0, 0, Int<0>{}, Int<NL>{});
  issue(1, 0, Int<NLA>{}, Int<NL>{}, 1);
  issue(1, 1, Int<0>{}, Int<NLA1>{});
  // slab 0 has landed once only slab 1's loads are in flight
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(NLA + NLA1) : "memory");
  read(w0, a0, wbuf(0), abuf(0), 0);
  int j = 0;
  for (; j + 6 <= nk; j += 6) static_for<0, 6>([&](auto it) {
    constexpr int i = decltype(it)::value;
    step(j + i, Int<i % 2>{}, Int<i % 3>{});
  });
  static_for<0, 5>([&](auto it) {
    constexpr int i = decltype(it)::value;
    if (j + i < nk) step(j + i, Int<i % 2>{}, Int<i % 3>{});
  });
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // epilogue: lane holds C[m][n] for m = m0 + 128 wm + 32 bm + l%32 and
  // n = n0 + 128 wn + 32 bn + 8g + 4(l/32) + e (accumulator slot 4g + e);
  // the bias of those columns is read now (8-byte loads where aligned and
  // inside N)
  u32x2 bias_pk[NB][4];
  {
    const bool bvec = ((uintptr_t)p.bias & 7u) == 0;
#pragma unroll
    for (int bn = 0; bn < NB; ++bn)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int nb = n0 + wn * WT + bn * 32 + 8 * g + 4 * fh;
        u32x2 v = {0u, 0u};
        if (p.bias) {
          if (bvec && nb + 3 < p.N) {
            v = *reinterpret_cast<const u32x2*>(p.bias + nb);
          } else {
            uint16_t h[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) h[e] = nb + e < p.N ? p.bias[nb + e] : (uint16_t)0;
            v[0] = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
            v[1] = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
          }
        }
        bias_pk[bn][g] = v;
      }
  }
  if ((p.N & 7) == 0) {
    // rows of C that are whole 16-byte chunks: every wave has read all of
    // the stages, so each takes one 32 KiB stage array for its 128 x 128
    // tile of C (rows of 256 bytes, 16-byte chunk c at c ^ (row & 15), so
    // that both the writes of 32 rows at one chunk and the reads of 4 whole
    // rows are free of bank conflicts) and stores it as whole rows: 16-byte
    // stores covering full 128-byte lines, marked non-temporal as C is not
    // read again.  (Stored straight from the accumulators, each store wrote
    // 16 bytes into each of 32 rows.)
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    char* ct = reinterpret_cast<char*>(wave == 0 ? as0 : wave == 1 ? as1 : wave == 2 ? ws0 : ws1);
#pragma unroll
    for (int bm = 0; bm < NB; ++bm)
#pragma unroll
      for (int bn = 0; bn < NB; ++bn)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint16_t bh = (uint16_t)(bias_pk[bn][g][e >> 1] >> (16 * (e & 1)));
            y[e] = gelu(acc[bn][bm][4 * g + e] + to_f32<BF16>(bh));
          }
          u32x2 v;
          v[0] = pack2<BF16>(y[0], y[1]);
          v[1] = pack2<BF16>(y[2], y[3]);
          const int r = bm * 32 + fr, cc = bn * 4 + g;
          *reinterpret_cast<u32x2*>(ct + r * 256 + ((cc ^ (r & 15)) << 4) + fh * 8) = v;
        }
#pragma unroll
    for (int i = 0; i < WT * WT * 2 / 1024; ++i) {
      const int lin = i * 64 + lane;
      const int r = lin >> 4, cc = lin & 15;
      const u32x4 v = *reinterpret_cast<const u32x4*>(ct + r * 256 + ((cc ^ (r & 15)) << 4));
      const int m = m0 + wm * WT + r, n = n0 + wn * WT + cc * 8;
      if (m < p.M && n < p.N) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p.c + (size_t)m * p.N + n));
    }
    return;
  }
  // otherwise straight from the accumulators
  const bool vec = (p.N & 3) == 0;
#pragma unroll
  for (int bm = 0; bm < NB; ++bm) {
    const int m = m0 + wm * WT + bm * 32 + fr;
    if (m >= p.M) continue;
    uint16_t* crow = p.c + (size_t)m * p.N;
#pragma unroll
    for (int bn = 0; bn < NB; ++bn)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int nb = n0 + wn * WT + bn * 32 + 8 * g + 4 * fh;
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint16_t bh = (uint16_t)(bias_pk[bn][g][e >> 1] >> (16 * (e & 1)));
          y[e] = gelu(acc[bn][bm][4 * g + e] + to_f32<BF16>(bh));
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
  // a work-group's buffer range (up to 256 rows of 2K bytes) and the tile
  // count stay inside 32 bits
  if ((int64_t)256 * K * 2 >= (int64_t)kOutOfRange) return FA_ERR_INVALID_ARG;
  const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
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
  const bool ktail = K % BK != 0;
  const void* fn = dtype == FA_BF16 ? (ktail ? reinterpret_cast<const void*>(&gemm_bias_gelu_kernel<true, true>)
                                             : reinterpret_cast<const void*>(&gemm_bias_gelu_kernel<true, false>))
                                    : (ktail ? reinterpret_cast<const void*>(&gemm_bias_gelu_kernel<false, true>)
                                             : reinterpret_cast<const void*>(&gemm_bias_gelu_kernel<false, false>));
  const hipError_t err = hipLaunchKernel(fn, dim3((unsigned)(tiles_m * tiles_n)), dim3(64 * kWaves), args, 0,
                                         static_cast<hipStream_t>(stream));
  return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}
