// fa_fwd.hip -- fused attention forward pass for gfx950 (MI355X), C ABI in fa.h.
//
// Method: the fused FlashAttention forward kernel of the TileLang tutorial
// pages (pro.edgex.exchange summary, paragraph on the fused FlashAttention
// forward kernel): Q, K and V are processed tile by tile, the full score
// matrix is never written to device memory, and the softmax is applied online
// with a running row maximum, a running normalising sum and rescale factors,
// both products running on the matrix cores.  Heads run in parallel and the
// keys of each head are streamed in order (comrad404.com, section "Как
// устроен туториал", FlashAttention paragraph).
//
// CDNA4 mapping.  One work-group of four waves owns (batch, head, 128
// queries); each wave owns 32 queries.  Two work-groups share a CU, so every
// SIMD runs two independent waves; registers stay within 256 per wave.
//
//  * Scores are formed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_{f16,bf16}: K (from LDS) is the A operand and the
//    wave's Q fragments (kept in VGPRs for the whole loop) are the B operand.
//    In the 32x32 accumulator layout a lane holds one column (one query) and
//    16 rows (keys), so each lane owns a query: row maximum and sum are
//    in-lane, plus one swap with the other half of the wave
//    (v_permlane32_swap).
//  * O is accumulated transposed, O^T = V^T P^T: the exponentiated scores,
//    packed to 16 bits in registers, are directly the B operand (a B
//    operand's lane layout equals the accumulator's column ownership).  The
//    V^T fragment is read from the V tile, kept in LDS in its natural
//    [key][d] layout, with ds_read_b64_tr_b16 (a transposing read: in each
//    16-lane group, lane i receives element i%4 of the 8-byte rows that lanes
//    i/4, i/4+4, i/4+8, i/4+12 point at).  The key order of a product's K
//    slots is free; the read addresses follow the order in which the
//    accumulator layout holds P.
//  * Software pipeline across key tiles: while the vector unit exponentiates
//    tile j, the matrix unit computes the scores of tile j+1 and the P.V
//    product of tile j, with the instructions interleaved so one wave keeps
//    both units busy.  K therefore runs one tile ahead of V in LDS: at tile j
//    the K tile j+1 and the V tile j are resident while K j+2 and V j+1
//    stream in.
//  * K and V tiles go from HBM straight into LDS (buffer_load_dwordx4 with
//    LDS destination: lane l of an instruction fills bytes 16l..16l+15 of a
//    1 KB block).  Each lane picks which 16-byte chunk of the tile it fetches,
//    which places the tile in LDS XOR-swizzled for the 64-bank LDS: K rows so
//    that the 16-byte fragment reads of 16 consecutive rows hit distinct
//    banks, V rows so that the transposing reads of 4 consecutive rows hit
//    distinct banks.  The buffer's range ends at the last key, so rows past
//    the end of the keys arrive as zeros.
//  * Online softmax with exp2 and scale*log2(e) folded into one FMA per
//    score.  Rescaling is lazy: a wave moves its reference maxima (and
//    rescales O and the sums) only when some row's maximum has grown by more
//    than 2^8 in exp2 units; otherwise the exponentials are taken against the
//    old reference and stay below 2^8, which 16-bit P holds at full relative
//    precision.  The reference cancels in O and is carried into lse.
//  * Tiles that need no mask run a branch-free path; tiles that cross the
//    causal diagonal or the end of the keys take the masked path; causal tiles
//    wholly above a wave's queries are skipped by that wave and never loaded
//    past the work-group's last query.
//  * Work-group ids are remapped so that the blocks of one head land on the
//    same XCD (each XCD has its own L2, and blocks of one head share K and V);
//    causal heads hand out their longest blocks first.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "fa.h"

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleLog2 = 8.0f;            // lazy-rescale threshold, exp2 units
constexpr uint32_t kBufferWord3 = 0x00020000u;  // raw buffer resource, gfx9 family
constexpr int kWaves = 4;                       // waves per work-group
constexpr int kBM = 32 * kWaves;                // queries per work-group

// scheduling-group masks of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedValu = 0x002;
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int Sq, Sk;
  int n_qblk;      // query blocks per (b, h)
  int n_wg;        // total work-groups
  float c;         // |scale| * log2(e)
  uint32_t qsign;  // 0x80008000 when scale < 0 (q is negated on load), else 0
  float cs;        // scale * log2(e), by which q is multiplied on load when pre-scaling
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

// Round two floats to the storage type (nearest even) and pack them.
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

// acc + (sum of the two fp16 values packed in w), accumulated in f32.
__device__ __forceinline__ float add_pair_f16(uint32_t w, float acc) {
  const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), one, acc, false);
}

// v_permlane32_swap exchanges the two 32-lane halves of a wave: afterwards
// the pair holds, in every lane, the values of lane l%32 and lane l%32+32.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                  __builtin_bit_cast(uint32_t, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                  __builtin_bit_cast(uint32_t, x), false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// max(a, b, c) as one v_max3_f32.  Written out because fmaxf would first
// quiet each input (the kernel runs with IEEE mode on), one extra instruction
// per input; a NaN score still reaches the output through its exponential.
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ __forceinline__ u32x4 lds_read_b128(const char* base, int off) {
  return *reinterpret_cast<const u32x4*>(base + off);
}

__device__ __forceinline__ u32x2 lds_read_tr16(const char* p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(u32x2, r);
}

// Work-group id -> logical block id.  Hardware hands consecutive ids to the
// 8 XCDs round-robin; this makes every XCD process one contiguous range of
// logical blocks (and so a few whole heads).
__device__ __forceinline__ int xcd_remap(int wg, int n) {
  const int xcd = wg & 7, local = wg >> 3;
  const int per = n >> 3, rem = n & 7;
  const int base = xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per;
  return base + local;
}

// LDS swizzles, in 16-byte chunks.  The LDS has 64 four-byte banks (256
// bytes); a 16-byte read by a wave is served 16 lanes at a time and a 8-byte
// transposing read 32 lanes at a time.
//  K: the score product's A fragment reads logical chunk c of 16 consecutive
//     rows in one pass; physical chunk c ^ ksw(row) puts them in 16 distinct
//     bank groups (D=64: two rows share a 256-byte bank line).
//  V: the transposing read covers 4 consecutive rows x 4 consecutive chunks
//     per pass; physical chunk c ^ vsw(row) spreads them over 16 groups.
template <int D>
__device__ __forceinline__ int ksw(int r) {
  return D == 64 ? ((r >> 1) & 7) : (r & 15);
}
template <int D>
__device__ __forceinline__ int vsw(int r) {
  return D == 64 ? ((r & 3) << 1) : ((r & 3) << 2);
}

// Stream NLD 1 KB blocks of one tensor's rows k0.. into LDS.  Lane l of
// block i fills bytes 16l..16l+15 of the block at dst + i*stride, reading the
// bytes at off[i] of the rows from key k0 on; the buffer range ends at key
// Sk, so rows past it arrive as zeros.
template <int NLD>
__device__ __forceinline__ void load_rows_to_lds(const uint16_t* g, int k0, int Sk, int rowb, char* dst,
                                                 int stride, const int* off) {
  const uint32_t bytes = (uint32_t)(Sk - k0) * (uint32_t)rowb;
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)g + (size_t)k0 * rowb), (short)0, bytes, kBufferWord3);
#pragma unroll
  for (int i = 0; i < NLD; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + i * stride), 16, off[i], 0, 0, 0);
}

template <bool B>
struct Flag { static constexpr bool value = B; };

template <int I>
struct Int { static constexpr int value = I; };

// s_waitcnt vmcnt(n) for n in {0, a, 2a, 3a, 4a} (the counter needs an immediate)
template <int A>
__device__ __forceinline__ void wait_vm(int n) {
  if (n <= 0)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else if (n <= A)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(A) : "memory");
  else if (n <= 2 * A)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * A) : "memory");
  else if (n <= 3 * A)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * A) : "memory");
  else
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * A) : "memory");
}

// PRE: q is multiplied by scale*log2(e) (rounded to fp16) when it is loaded,
// so the score products give exp2-domain logits directly, and the scores a
// step exponentiates are kept relative to the row's reference.  A row's
// first reference is 0 when its first maximum lies within +-kRescaleLog2 of
// 0 (moderate logits); while every row of a wave has the reference 0,
// P = exp2(s) needs no subtraction at all.
template <int D, bool BF16, bool CAUSAL, int BN, bool PRE>
__global__ __launch_bounds__(256, 2) void fa_fwd_kernel(Params p) {
  constexpr int CH = D / 8;                       // 16-byte chunks per row
  constexpr int ROWB = 2 * D;                     // bytes per row
  constexpr int TILE = BN * ROWB;                 // bytes of one K or V tile
  constexpr int NLD = TILE / 16 / (64 * kWaves);  // load instructions per wave per tile
  constexpr int KB = BN / 32;                     // 32-key blocks per tile
  constexpr int NU = BN / 16;                     // 16-key slices per tile (P.V product steps)
  constexpr int DK = D / 16;                      // k-steps of the score product
  constexpr int DB = D / 32;                      // 32-wide d blocks of the output
  constexpr int NS = KB * DK;                     // score products per tile
  constexpr int NSA = NS / 2;                     // of which issued ahead of the row maximum
  static_assert(TILE % (16 * 64 * kWaves) == 0, "tile must split evenly over the waves");
  static_assert(!(PRE && BF16), "pre-scaling rounds q to fp16");
  static_assert(DK >= NSA, "the early score products must share one 32-key block");

  // A ring of four LDS stages per tensor (tile t in stage t % 4), each a
  // separate array: the compiler can then tell that the loads streaming into
  // one stage never alias the reads from another.  Tiles are loaded two steps
  // before they are read, which hides the load latency of a step.
  __shared__ u32x4 kst0[TILE / 16];
  __shared__ u32x4 kst1[TILE / 16];
  __shared__ u32x4 kst2[TILE / 16];
  __shared__ u32x4 kst3[TILE / 16];
  __shared__ u32x4 vst0[TILE / 16];
  __shared__ u32x4 vst1[TILE / 16];
  __shared__ u32x4 vst2[TILE / 16];
  __shared__ u32x4 vst3[TILE / 16];
  auto kbuf = [&](int t) -> char* {
    return reinterpret_cast<char*>(t == 0 ? kst0 : t == 1 ? kst1 : t == 2 ? kst2 : kst3);
  };
  auto vbuf = [&](int t) -> char* {
    return reinterpret_cast<char*>(t == 0 ? vst0 : t == 1 ? vst1 : t == 2 ? vst2 : vst3);
  };

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps per-wave branches scalar
  const int lane = tid & 63;
  const int n = lane & 31;  // query column owned by this lane
  const int h = lane >> 5;  // which half of the wave

  const int t = xcd_remap(blockIdx.x, p.n_wg);
  const int bh = t / p.n_qblk;
  int qblk = t - bh * p.n_qblk;
  if (CAUSAL) qblk = p.n_qblk - 1 - qblk;  // longest blocks first
  const int q0 = qblk * kBM;
  const int qw0 = q0 + wave * 32;  // first query of this wave
  const int qi = qw0 + n;          // query of this lane

  const uint16_t* qg = p.q + (size_t)bh * p.Sq * D;
  const uint16_t* kg = p.k + (size_t)bh * p.Sk * D;
  const uint16_t* vg = p.v + (size_t)bh * p.Sk * D;

  const int kend = CAUSAL ? min(p.Sk, q0 + kBM) : p.Sk;
  const int ntiles = (kend + BN - 1) / BN;
  // tiles this wave computes: all of the work-group's, less (causal) those
  // wholly above its last query; none for waves past the last query
  int nt_w = CAUSAL ? min(ntiles, (qw0 + 31) / BN + 1) : ntiles;
  if (qw0 >= p.Sq) nt_w = 0;
  // the first tile that needs a mask: the one holding the end of the keys
  // (when Sk is not a multiple of BN) or, causal, the first that reaches past
  // this wave's first query
  int j_mask = p.Sk / BN;
  if (CAUSAL) j_mask = min(j_mask, (qw0 + 1) / BN);
  // tiles 0 .. j_fast-1 need no mask and have a successor: the branch-free
  // loop runs them in pairs
  // (and the loads they issue, two tiles ahead, all exist: the loop waits
  // for them with a fixed count)
  const int j_fast = max(0, min(min(nt_w - 1, j_mask), ntiles - 3)) & ~3;

  // ---- tile loads: each lane fetches the global chunk that belongs at its LDS slot
  int offk[NLD], offv[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int slot = (i * kWaves + wave) * 64 + lane;  // 16-byte slot within the tile
    const int r = slot / CH, pc = slot % CH;
    offk[i] = r * ROWB + ((pc ^ ksw<D>(r)) << 4);
    offv[i] = r * ROWB + ((pc ^ vsw<D>(r)) << 4);
  }
  auto issue_k = [&](int tile, char* buf) {
    load_rows_to_lds<NLD>(kg, tile * BN, p.Sk, ROWB, buf + wave * 1024, kWaves * 1024, offk);
  };
  auto issue_v = [&](int tile, char* buf) {
    load_rows_to_lds<NLD>(vg, tile * BN, p.Sk, ROWB, buf + wave * 1024, kWaves * 1024, offv);
  };

  // K 0 first (the prologue's scores need it), then K 1, V 0, K 2, V 1
  issue_k(0, kbuf(0));
  int loads_after_k0 = 0;
  if (ntiles > 1) { issue_k(1, kbuf(1)); loads_after_k0 += NLD; }
  issue_v(0, vbuf(0));
  loads_after_k0 += NLD;
  if (ntiles > 2) { issue_k(2, kbuf(2)); loads_after_k0 += NLD; }
  if (ntiles > 1) { issue_v(1, vbuf(1)); loads_after_k0 += NLD; }

  // ---- Q fragments: B operands of S^T = K Q^T; lane holds q[qi][16*ks + 8*h .. +8]
  u32x4 qf[DK];
#pragma unroll
  for (int ks = 0; ks < DK; ++ks) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (qi < p.Sq) x = *reinterpret_cast<const u32x4*>(qg + (size_t)qi * D + ks * 16 + h * 8);
    if constexpr (PRE) {
      f16x8 v = __builtin_bit_cast(f16x8, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (_Float16)((float)v[e] * p.cs);
      x = __builtin_bit_cast(u32x4, v);
    } else {
      x ^= p.qsign;
    }
    qf[ks] = x;
  }

  // ---- per-lane fragment read offsets (bytes within a tile)
  // K (A operand of S^T): row 32*kb + n, logical chunk 2*ks + h.
  int koff[DK];
#pragma unroll
  for (int ks = 0; ks < DK; ++ks) koff[ks] = n * ROWB + (((2 * ks + h) ^ ksw<D>(n)) << 4);
  // V (A operand of O^T through the transposing read): in 16-lane group g
  // (lane = 16g + s) source lane s points at row 4*(g/2) + s/4 (+ 16u + 8*half)
  // and element 32*db + 16*(g%2) + 4*(s%4); the lane then receives
  // d = 32*db + lane%32 for keys 16u + 8*half + 4*h + (0..3).
  const int g = lane >> 4, s = lane & 15;
  const int vrow = 4 * (g >> 1) + (s >> 2);
  int voff[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int chunk = 4 * db + 2 * (g & 1) + ((s & 3) >> 1);
    voff[db] = vrow * ROWB + ((chunk ^ vsw<D>(vrow)) << 4) + ((s & 1) << 3);
  }

  // ---- running state of this lane's query
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  // reference maximum of the scores: raw units, or exp2 units when PRE
  float m_ref = -INFINITY;
  float l_run = 0.f;        // this half's share of the running normaliser
  const float c = PRE ? 1.f : p.c;  // score -> exp2 units
  bool zero_ref = true;     // PRE: every row of the wave has the reference 0 (or none yet)

  // i-th score product of a tile: S^T[32kb.., q] += K[32kb + n][16ks + 8h ..] q[..]
  auto score_mfma = [&](f32x16* sacc, const char* kt, int i) {
    const int kb = i / DK, ks = i % DK;
    sacc[kb] = mfma_32x32x16<BF16>(lds_read_b128(kt, koff[ks] + kb * 32 * ROWB), qf[ks], sacc[kb]);
  };

  // One key tile: softmax and P.V of tile j (scores in sacc, V tile at vt),
  // and, when NEXT, the scores of tile j+1 into snext from the K tile at kn.
  // sacc[kb][r] = score(query qi, key k0 + 32kb + 8(r/4) + 4h + r%4).
  auto tile_step = [&](f32x16* sacc, f32x16* snext, const char* kn, const char* vt, int k0, auto mask_tag,
                       auto next_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr bool NEXT = decltype(next_tag)::value;

    // the first half of the next tile's score products runs under the row max
    if constexpr (NEXT) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) snext[kb][r] = 0.f;
#pragma unroll
      for (int i = 0; i < NSA; ++i) score_mfma(snext, kn, i);
    }

    if constexpr (PRE) {
      // scores relative to the reference (nothing to do while it is 0)
      if (!zero_ref) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[kb][r] -= m_ref;
      }
    }
    if constexpr (MASK) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (key >= p.Sk || (CAUSAL && key > qi)) sacc[kb][r] = -INFINITY;
        }
    }

    // tile row max (both halves of the wave), in two independent chains
    float m2[2] = {sacc[0][0], sacc[0][1]};
#pragma unroll
    for (int i = 2; i < 16 * KB; i += 2)
      m2[(i >> 1) & 1] = max3(m2[(i >> 1) & 1], sacc[i >> 4][i & 15], sacc[i >> 4][(i & 15) + 1]);
    const float mx = max_halves(fmaxf(m2[0], m2[1]));

    // lazy rescale: move the reference only when some row's max grew past the threshold
    if constexpr (PRE) {
      const bool first = m_ref == -INFINITY;
      const bool grow = first || mx > kRescaleLog2;
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        // shift of this row's reference, relative to the scores in sacc
        const float delta = first ? (fabsf(mx) <= kRescaleLog2 ? 0.f : mx) : (grow ? mx : 0.f);
        const float alpha = first ? 0.f : exp2f(-delta);
        m_ref = first ? delta : m_ref + delta;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        if (__builtin_amdgcn_ballot_w64(delta != 0.f) != 0) {
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[kb][r] -= delta;
        }
        zero_ref = __builtin_amdgcn_ballot_w64(m_ref != 0.f) == 0;
      }
    } else {
      const bool grow = (m_ref == -INFINITY) || ((mx - m_ref) * c > kRescaleLog2);
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        const float m_new = fmaxf(m_ref, mx);
        const float alpha = (m_ref == -INFINITY) ? 0.f : exp2f((m_ref - m_new) * c);
        m_ref = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      }
    }
    const float mc = m_ref * c;

    // P = exp2(s*c - m*c), packed to 16 bits; running sum
    u32x4 pf[NU];
    float psum = l_run;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      float pv[8];
#pragma unroll
      for (int t8 = 0; t8 < 8; ++t8) {
        const float sv = sacc[u >> 1][8 * (u & 1) + t8];
        float pe;
        if constexpr (PRE)
          pe = __builtin_amdgcn_exp2f(sv);  // relative scores, exp2 units
        else
          pe = __builtin_amdgcn_exp2f(__builtin_fmaf(sv, c, -mc));
        if constexpr (MASK && !PRE) pe = (sv == -INFINITY) ? 0.f : pe;  // also covers scale == 0
        pv[t8] = pe;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pf[u][e] = pack2<BF16>(pv[2 * e], pv[2 * e + 1]);
        // fp16 rounds P to within 2^-12, so summing the rounded values keeps the
        // normaliser (and lse) accurate; bf16 rounding (2^-9) would not, so bf16
        // sums the fp32 values.
        if constexpr (BF16)
          psum += pv[2 * e] + pv[2 * e + 1];
        else
          psum = add_pair_f16(pf[u][e], psum);
      }
    }
    l_run = psum;

    // O^T += V^T P^T
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const char* vp = vt + voff[db] + 16 * u * ROWB;
        const u32x2 lo = lds_read_tr16(vp);
        const u32x2 hi = lds_read_tr16(vp + 8 * ROWB);
        const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
        oacc[db] = mfma_32x32x16<BF16>(a, pf[u], oacc[db]);
      }

    // the second half of the next tile's score products
    if constexpr (NEXT) {
#pragma unroll
      for (int i = NSA; i < NS; ++i) score_mfma(snext, kn, i);
    }

    // Interleave: one matrix instruction, then a run of vector instructions
    // and LDS reads, so the wave keeps the matrix unit busy while it
    // exponentiates.
    constexpr int NMF = NU * DB + (NEXT ? NS - NSA : 0);
    constexpr int NVALU = NU * (8 + 8 + 4 + (BF16 ? 8 : 4));
    constexpr int VPM = (NVALU + NMF - 1) / NMF;
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
#pragma unroll
    for (int i = 0; i < NMF; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedValu, VPM, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
    }
  };

  // Step j reads K tile j+1 and V tile j, loaded at step j-2 (or before the
  // loop): after the wait, the barrier makes them visible to every wave and
  // guarantees that every wave is done with K tile j-1 and V tile j-2, whose
  // stages take K tile j+3 and V tile j+2.
  auto issue_next = [&](int j) {
    if (j + 3 < ntiles) issue_k(j + 3, kbuf((j + 3) & 3));
    if (j + 2 < ntiles) issue_v(j + 2, vbuf((j + 2) & 3));
  };
  // branch-free step (compile-time stages): the previous step issued 2*NLD loads
  auto step_fast = [&](int j, auto jm4_tag, f32x16* sacc, f32x16* snext) {
    constexpr int jm = decltype(jm4_tag)::value;  // j % 4
    // the wait and the barrier in one asm statement with a memory clobber:
    // no LDS access moves across it, and no release fence makes the compiler
    // wait for the loads still in flight (they target other stages); every
    // LDS read of the previous step has returned (lgkmcnt) before any wave
    // may overwrite its stage
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * NLD) : "memory");
    __builtin_amdgcn_sched_barrier(0);
    issue_k(j + 3, kbuf((jm + 3) & 3));
    issue_v(j + 2, vbuf((jm + 2) & 3));
    tile_step(sacc, snext, kbuf((jm + 1) & 3), vbuf(jm), j * BN, Flag<false>{}, Flag<true>{});
  };
  // any tile: masked or not, with or without a successor; the scores of the
  // successor land in snext and are moved to sacc
  auto step = [&](int j, f32x16* sacc, f32x16* snext) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    issue_next(j);
    if (j < nt_w) {
      const char* knext = kbuf((j + 1) & 3);
      const char* vcur = vbuf(j & 3);
      // the few tiles past the branch-free loop all take the masked path
      // (the mask is exact for any tile), which keeps this loop small
      const int k0 = j * BN;
      if (j + 1 < nt_w)
        tile_step(sacc, snext, knext, vcur, k0, Flag<true>{}, Flag<true>{});
      else
        tile_step(sacc, snext, knext, vcur, k0, Flag<true>{}, Flag<false>{});
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) sacc[kb] = snext[kb];
    }
  };

  // scores of tile 0
  f32x16 sa[KB], sb[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) sa[kb][r] = 0.f;
  wait_vm<NLD>(loads_after_k0);  // K tile 0 has landed
  __syncthreads();
  if (nt_w > 0) {
#pragma unroll
    for (int i = 0; i < NS; ++i) score_mfma(sa, kbuf(0), i);
  }

  // (the fast loop's first step waits for all but 2*NLD loads: K 2 and V 1
  // may still be in flight, K 1 and V 0 have landed)
  int j = 0;
  for (; j < j_fast; j += 4) {
    step_fast(j, Int<0>{}, sa, sb);
    step_fast(j + 1, Int<1>{}, sb, sa);
    step_fast(j + 2, Int<2>{}, sa, sb);
    step_fast(j + 3, Int<3>{}, sb, sa);
  }
  for (; j < ntiles; ++j) step(j, sa, sb);

  // ---- epilogue: normalise, round, store O rows and lse
  if (qw0 < p.Sq) {
    const float l = sum_halves(l_run);
    if (qi < p.Sq) {
      const float inv = 1.f / l;
      uint16_t* og = p.o + ((size_t)bh * p.Sq + qi) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int d0 = db * 32 + 8 * gq + 4 * h;
          u32x2 w;
          w[0] = pack2<BF16>(oacc[db][4 * gq] * inv, oacc[db][4 * gq + 1] * inv);
          w[1] = pack2<BF16>(oacc[db][4 * gq + 2] * inv, oacc[db][4 * gq + 3] * inv);
          *reinterpret_cast<u32x2*>(og + d0) = w;
        }
      if (h == 0) p.lse[(size_t)bh * p.Sq + qi] = (m_ref * c + __log2f(l)) * kLn2;  // c = 1 when PRE
    }
  }
}

// Keys per tile for each (head dim, dtype, mask).
template <int D, bool BF16, bool CAUSAL>
struct Cfg {
  static constexpr int BN = D == 64 ? 64 : 32;
};

template <int D, bool BF16, bool CAUSAL>
hipError_t launch(const Params& base, int64_t BH, int64_t Sq, hipStream_t stream) {
  using C = Cfg<D, BF16, CAUSAL>;
  Params p = base;
  p.n_qblk = (int)((Sq + kBM - 1) / kBM);
  p.n_wg = (int)(BH * p.n_qblk);
  void* args[] = {&p};
  // pre-scale fp16 q when |scale*log2(e)| <= 1, so q*scale*log2(e) cannot overflow
  const void* fn = reinterpret_cast<const void*>(&fa_fwd_kernel<D, BF16, CAUSAL, C::BN, false>);
  if constexpr (!BF16)
    if (fabsf(p.cs) <= 1.f) fn = reinterpret_cast<const void*>(&fa_fwd_kernel<D, BF16, CAUSAL, C::BN, true>);
  return hipLaunchKernel(fn, dim3(p.n_wg), dim3(64 * kWaves), args, 0, stream);
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

}  // namespace

extern "C" fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                            int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                            float scale, int causal, int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if ((((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u) || ((uintptr_t)lse & 3u))
    return FA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || Sq < 1 || Sk < 1 || D < 1) return FA_ERR_INVALID_ARG;
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
  if (!isfinite(scale)) return FA_ERR_INVALID_ARG;
  const int64_t lim = (int64_t)1 << 31;
  if (Sq >= lim / D || Sk >= lim / D) return FA_ERR_INVALID_ARG;
  if (B >= lim / H) return FA_ERR_INVALID_ARG;
  const int64_t BH = B * H;
  const int64_t minBM = kBM;  // queries per work-group
  if (BH >= lim / ((Sq + minBM - 1) / minBM)) return FA_ERR_INVALID_ARG;
  // element counts in int64: BH < 2^31 and S*D < 2^31 keep these below 2^62
  const size_t qo_bytes = (size_t)(BH * Sq * D) * 2, kv_bytes = (size_t)(BH * Sk * D) * 2;
  const size_t lse_bytes = (size_t)(BH * Sq) * 4;
  if (overlaps(o, qo_bytes, q, qo_bytes) || overlaps(o, qo_bytes, k, kv_bytes) ||
      overlaps(o, qo_bytes, v, kv_bytes) || overlaps(lse, lse_bytes, q, qo_bytes) ||
      overlaps(lse, lse_bytes, k, kv_bytes) || overlaps(lse, lse_bytes, v, kv_bytes) ||
      overlaps(o, qo_bytes, lse, lse_bytes))
    return FA_ERR_INVALID_ARG;

  Params p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.Sq = (int)Sq;
  p.Sk = (int)Sk;
  p.n_qblk = 0;
  p.n_wg = 0;
  p.c = (float)(fabs((double)scale) * 1.4426950408889634);
  p.qsign = scale < 0.f ? 0x80008000u : 0u;
  p.cs = (float)((double)scale * 1.4426950408889634);

  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf = dtype == FA_BF16;
  hipError_t err;
  if (D == 64) {
    if (bf) err = causal ? launch<64, true, true>(p, BH, Sq, s) : launch<64, true, false>(p, BH, Sq, s);
    else err = causal ? launch<64, false, true>(p, BH, Sq, s) : launch<64, false, false>(p, BH, Sq, s);
  } else {
    if (bf) err = causal ? launch<128, true, true>(p, BH, Sq, s) : launch<128, true, false>(p, BH, Sq, s);
    else err = causal ? launch<128, false, true>(p, BH, Sq, s) : launch<128, false, false>(p, BH, Sq, s);
  }
  return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

extern "C" const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARG: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported head dimension or dtype";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}
