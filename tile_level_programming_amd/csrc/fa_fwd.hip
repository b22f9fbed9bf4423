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
// queries); each wave owns 32 queries.  Key tiles are 32 keys long.  At
// D=64 three work-groups share a CU (registers within 168 per wave), at
// D=128 two (within 256), so every SIMD runs three or two independent waves.
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
//  * Software pipeline across key tiles, three deep: step j runs the score
//    products of tile j+2 and the P.V product of tile j on the matrix unit,
//    interleaved with the exponentials of tile j+1 on the vector unit; the
//    two streams share no data.  K tiles run two ahead of V in LDS, in a
//    ring of four stages per tensor, and the K fragments of a step are read
//    from LDS by the step before.
//  * K and V tiles go from HBM straight into LDS (buffer_load_dwordx4 with
//    LDS destination: lane l of an instruction fills bytes 16l..16l+15 of a
//    1 KB block).  Each lane picks which 16-byte chunk of the tile it fetches,
//    which places the tile in LDS XOR-swizzled for the 64-bank LDS: K rows so
//    that the 16-byte fragment reads of 16 consecutive rows hit distinct
//    banks, V rows so that the transposing reads of 4 consecutive rows hit
//    distinct banks.  The buffer's range ends at the last key, so rows past
//    the end of the keys arrive as zeros.
//  * Online softmax with exp2 (scale*log2(e) applied as one multiply per
//    score) against a per-row reference m.  The score products start from
//    -m, so the scores come out relative to it at no cost.  The reference
//    is the first tile's row maximum and moves only when a tile's P grows
//    large (a row's sum over the tile above a bound): then O and the sums
//    are rescaled and the tile is exponentiated again.  No per-tile row
//    maximum is taken otherwise.  The reference cancels in O and is carried
//    into lse.  The branch-free steps take the row sums of the packed P on
//    the matrix unit (a 0/1 operand), which keeps 32 additions per lane and
//    tile off the vector unit.
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

#include <mutex>

#include "fa.h"

// Fixed device buffer of fa_fwd_split_noalloc: the partial results of the
// key split live here instead of in a caller workspace.  Each device the
// library runs on holds its own copy until the process ends.  In host code
// this name is only a handle for hipGetSymbolAddress; the device address is
// looked up once per device (scratch_on_current_device) and passed to the
// kernels like any workspace.
static __device__ __align__(256) unsigned char scratch[FA_SPLIT_SCRATCH_BYTES];

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLn2 = 0.6931471805599453f;
// A row's sum of P over one tile above this makes its wave move the
// reference (and rescale); below it every P of the tile is at most this,
// far inside the 16-bit range (fp16 max 65504).
constexpr float kSumBound = 4096.0f;
constexpr uint32_t kBufferWord3 = 0x00020000u;  // raw buffer resource, gfx9 family
constexpr int kWaves = 4;                       // waves per work-group
constexpr int kBM = 32 * kWaves;                // queries per work-group (one key group)

// scheduling-group masks of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedValu = 0x002;
constexpr int kSchedMfma = 0x008;
constexpr int kSchedVmem = 0x010;
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
  int xcd_heads;   // causal, no split: heads per XCD when every XCD gets whole heads, else 0
  float c;         // |scale| * log2(e), at least 1e-30
  uint32_t qsign;  // 0x80008000 when scale < 0 (q is negated on load), else 0
  // split over the keys: range r holds keys r*kchunk .. min(Sk, (r+1)*kchunk)-1
  int n_split;     // ranges (1 without a split)
  int kchunk;      // keys per range, a multiple of 64
  int n_bh;        // B*H
  float* po;       // partial O, fp32 [n_split][B*H*Sq][D], normalised over the range
  float* plse;     // partial lse, fp32 [n_split][B*H*Sq]
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
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 acc) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
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

// The two 16-bit values of a packed pair, back in fp32 (exact), added: the
// normaliser that divides O is the sum of the same rounded P that the P.V
// product multiplies, so O is a convex combination of the V rows with the
// rounded weights.
template <bool BF16>
__device__ __forceinline__ float sum_pair(uint32_t x) {
  if constexpr (BF16) {
    return __builtin_bit_cast(float, x << 16) + __builtin_bit_cast(float, x & 0xffff0000u);
  } else {
    const f16x2 h = __builtin_bit_cast(f16x2, x);
    return (float)h[0] + (float)h[1];
  }
}

// v_permlane32_swap exchanges the two 32-lane halves of a wave: afterwards
// the pair holds, in every lane, the values of lane l%32 and lane l%32+32.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                  __builtin_bit_cast(uint32_t, x), false, false);
  return __builtin_elementwise_maximum(__builtin_bit_cast(float, (uint32_t)r[0]),
                                       __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                  __builtin_bit_cast(uint32_t, x), false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// max(a, b, c) with NaN propagation (IEEE 754-2019 maximum): one
// v_maximum3_f32, with no quieting of the inputs that fmaxf would need in
// IEEE mode.  A NaN score makes its row's maximum, and so its output, NaN.
__device__ __forceinline__ float max3(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
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
// bytes at off[i] of the rows from key k0 on.  `r` is one buffer resource
// for the whole key range, made once: the tile's start goes into each lane's
// offset, so the range check (offset below the range's size) zero-fills the
// rows past the last key and a tile wholly past the keys touches no memory.
// Its loads still count in vmcnt, which keeps the number of loads in flight
// the same every step.  The offsets are 32-bit: K and V are below 2^32 bytes
// per head (Sk*D < 2^31), and an offset of a tile past the end that wraps
// lands inside the range, where it reads real rows into a stage no product
// uses.
template <int NLD>
__device__ __forceinline__ void load_rows_to_lds(__amdgpu_buffer_rsrc_t r, int k0, int rowb, char* dst, int stride,
                                                 const int* off) {
  const uint32_t base = (uint32_t)k0 * (uint32_t)rowb;
#pragma unroll
  for (int i = 0; i < NLD; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + i * stride), 16, (int)(base + (uint32_t)off[i]),
                                             0, 0, 0);
}

template <int I>
struct Int { static constexpr int value = I; };

// KG key groups of kWaves/KG waves each (1, or 2 for launches that leave
// most CUs idle): group g takes the g-th share of the block's key tiles, the
// groups' partial results are merged through LDS at the end, and a
// work-group owns 32*kWaves/KG queries.  The longest block's work is then
// spread over KG times as many work-groups, each SIMD doing 1/KG of it.
template <int D, bool BF16, bool CAUSAL, int BN, bool SPLIT, int KG = 1>
__global__ __launch_bounds__(256, KG == 2 ? 1 : D == 64 && BN == 32 ? 3 : 2) void fa_fwd_kernel(Params p) {
  constexpr int WPG = kWaves / KG;                // waves per key group
  constexpr int BM = 32 * WPG;                    // queries per work-group
  constexpr int CH = D / 8;                       // 16-byte chunks per row
  constexpr int ROWB = 2 * D;                     // bytes per row
  constexpr int TILE = BN * ROWB;                 // bytes of one K or V tile
  constexpr int NLD = TILE / 16 / (64 * WPG);     // load instructions per wave per tile
  constexpr int KB = BN / 32;                     // 32-key blocks per tile
  constexpr int NU = BN / 16;                     // 16-key slices per tile (P.V product steps)
  constexpr int DK = D / 16;                      // k-steps of the score product
  constexpr int DB = D / 32;                      // 32-wide d blocks of the output
  constexpr int NS = KB * DK;                     // score products per tile
  constexpr int NSA = NS / 2;                     // of which issued ahead of the row maximum
  static_assert(TILE % (16 * 64 * WPG) == 0, "tile must split evenly over the waves");
  static_assert(KG == 1 || (KG == 2 && !SPLIT), "two key groups only without a split over the keys");
  static_assert(DK >= NSA, "the early score products must share one 32-key block");

  // A ring of four LDS stages per tensor (tile t in stage t % 4), each a
  // separate array: the compiler can then tell that the loads streaming into
  // one stage never alias the reads from another.  Tiles are loaded two steps
  // before they are read, which hides the load latency of a step.
  // (With two key groups each stage holds one tile per group.)
  __shared__ u32x4 kst0[KG * TILE / 16];
  __shared__ u32x4 kst1[KG * TILE / 16];
  __shared__ u32x4 kst2[KG * TILE / 16];
  __shared__ u32x4 kst3[KG * TILE / 16];
  __shared__ u32x4 vst0[KG * TILE / 16];
  __shared__ u32x4 vst1[KG * TILE / 16];
  __shared__ u32x4 vst2[KG * TILE / 16];
  __shared__ u32x4 vst3[KG * TILE / 16];

  const int tid = threadIdx.x;
  // the wave within its key group, and the group (uniform: keeps per-wave
  // branches scalar)
  const int wave = __builtin_amdgcn_readfirstlane((tid >> 6) % WPG);
  const int grp = KG == 1 ? 0 : __builtin_amdgcn_readfirstlane((tid >> 6) / WPG);
  const int lane = tid & 63;
  auto kbuf = [&](int t) __attribute__((always_inline)) -> char* {
    return reinterpret_cast<char*>(t == 0 ? kst0 : t == 1 ? kst1 : t == 2 ? kst2 : kst3) + grp * TILE;
  };
  auto vbuf = [&](int t) __attribute__((always_inline)) -> char* {
    return reinterpret_cast<char*>(t == 0 ? vst0 : t == 1 ? vst1 : t == 2 ? vst2 : vst3) + grp * TILE;
  };
  // The fragment reads of stage t.  With two key groups they take the stage's
  // base (a constant, which the LDS reads carry as their immediate offset)
  // and the group's offset sits in the per-lane offsets koff and voff: a
  // runtime base per stage would cost a register per stage and fragment,
  // and would hide from the compiler which stage a read touches, so that it
  // waited for every load in flight (they write other stages) before reads.
  constexpr int GOFF = KG > 1 ? TILE : 0;  // per-lane offset of group 1's tiles
  auto krd = [&](int t) __attribute__((always_inline)) -> const char* {
    if constexpr (KG == 1) return kbuf(t);
    else return reinterpret_cast<const char*>(t == 0 ? kst0 : t == 1 ? kst1 : t == 2 ? kst2 : kst3);
  };
  auto vrd = [&](int t) __attribute__((always_inline)) -> const char* {
    if constexpr (KG == 1) return vbuf(t);
    else return reinterpret_cast<const char*>(t == 0 ? vst0 : t == 1 ? vst1 : t == 2 ? vst2 : vst3);
  };
  const int n = lane & 31;  // query column owned by this lane
  const int h = lane >> 5;  // which half of the wave

  // logical block t = (bh * n_split + range) * n_qblk + query block: the
  // query blocks that read the same keys are neighbours
  int qblk, split, bh;
  if (CAUSAL && !SPLIT && p.xcd_heads > 0) {
    // Every XCD owns xcd_heads whole heads (their keys stay in its L2) and
    // runs its blocks longest first across all of them: its work-groups
    // then finish together.  Head by head, longest first within each head,
    // the long blocks of its last heads would start late.
    const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    const int rank = local / p.xcd_heads;  // 0: the longest blocks
    bh = xcd * p.xcd_heads + (local - rank * p.xcd_heads);
    qblk = p.n_qblk - 1 - rank;
    split = 0;
  } else {
    const int t = xcd_remap(blockIdx.x, p.n_wg);
    const int t2 = t / p.n_qblk;
    qblk = t - t2 * p.n_qblk;
    split = SPLIT ? t2 % p.n_split : 0;
    bh = SPLIT ? t2 / p.n_split : t2;
    if (CAUSAL) qblk = p.n_qblk - 1 - qblk;  // longest blocks first
  }
  const int q0 = qblk * BM;
  const int qw0 = q0 + wave * 32;  // first query of this wave
  const int qi = qw0 + n;          // query of this lane

  // the keys of this block: all of them, or (split) the Skl keys from kb0 on,
  // or (two key groups) group g's share of the block's key tiles, tpg tiles
  // from tile g*tpg on; tiles, masks and loads count keys from kb0
  const int kend0 = CAUSAL ? min(p.Sk, q0 + BM) : p.Sk;  // (two key groups) the block's keys
  const int tpg = KG == 1 ? 0 : ((kend0 + BN - 1) / BN + KG - 1) / KG;
  const int kb0 = SPLIT ? split * p.kchunk : KG == 1 ? 0 : grp * tpg * BN;
  const int Skl = SPLIT ? min(p.Sk - kb0, p.kchunk) : KG == 1 ? p.Sk : max(0, min(p.Sk - kb0, tpg * BN));
  const int qw0r = qw0 - kb0;  // query positions relative to kb0 (the causal
  const int qir = qi - kb0;    // mask compares them with key positions)

  const uint16_t* qg = p.q + (size_t)bh * p.Sq * D;
  const uint16_t* kg = p.k + ((size_t)bh * p.Sk + kb0) * D;
  const uint16_t* vg = p.v + ((size_t)bh * p.Sk + kb0) * D;

  const int kend = CAUSAL ? min(Skl, q0 - kb0 + BM) : Skl;  // (split, key groups, causal: may be <= 0)
  const int ntiles = kend > 0 ? (kend + BN - 1) / BN : 0;
  // steps of every wave of the work-group (each step has one barrier)
  const int nsteps = KG == 1 ? ntiles : tpg;
  // tiles this wave computes: all of the work-group's, less (causal) those
  // wholly above its last query; none for waves past the last query
  int nt_w = CAUSAL ? (qw0r + 31 < 0 ? 0 : min(ntiles, (qw0r + 31) / BN + 1)) : ntiles;
  if (qw0 >= p.Sq) nt_w = 0;
  // the first tile that needs a mask: the one holding the end of the keys
  // (when Skl is not a multiple of BN) or, causal, the first that reaches
  // past this wave's first query
  int j_mask = Skl / BN;
  if (CAUSAL) j_mask = min(j_mask, qw0r + 1 <= 0 ? 0 : (qw0r + 1) / BN);
  // steps 0 .. j_fast-1 run branch-free: step j exponentiates tile j+1
  // (which must need no mask) and forms the scores of tile j+2 (which must
  // exist); a multiple of 4 steps, one per LDS stage
  const int j_fast = max(0, min(j_mask - 1, nt_w - 2)) & ~3;

  // ---- tile loads: each lane fetches the global chunk that belongs at its LDS slot
  int offk[NLD], offv[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int slot = (i * WPG + wave) * 64 + lane;  // 16-byte slot within the tile
    const int r = slot / CH, pc = slot % CH;
    offk[i] = r * ROWB + ((pc ^ ksw<D>(r)) << 4);
    offv[i] = r * ROWB + ((pc ^ vsw<D>(r)) << 4);
  }
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc((void*)kg, (short)0, (uint32_t)Skl * ROWB, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc((void*)vg, (short)0, (uint32_t)Skl * ROWB, kBufferWord3);
  auto issue_k = [&](int tile, char* buf) __attribute__((always_inline)) {
    load_rows_to_lds<NLD>(rk, tile * BN, ROWB, buf + wave * 1024, WPG * 1024, offk);
  };
  auto issue_v = [&](int tile, char* buf) __attribute__((always_inline)) {
    load_rows_to_lds<NLD>(rv, tile * BN, ROWB, buf + wave * 1024, WPG * 1024, offv);
  };

  // ---- Q fragments: B operands of S^T = K Q^T; lane holds q[qi][16*ks + 8*h .. +8].
  // Loaded before the tiles: the load counter drains in order, so Q issued
  // after them would wait for every tile of the prologue.  Every lane loads
  // (rows past the queries read the last row, Sq >= 1) and those rows are
  // zeroed once the tiles are issued: a load under a branch per lane let
  // the compiler wait for it inside the branch, before the tiles went out.
  u32x4 qf[DK];
  const int qrow = min(qi, p.Sq - 1);
#pragma unroll
  for (int ks = 0; ks < DK; ++ks) qf[ks] = *reinterpret_cast<const u32x4*>(qg + (size_t)qrow * D + ks * 16 + h * 8);

  // Tile t of K lands two steps before its fragments are read (at the end of
  // step t-3), tile t of V three steps before it is read (step t): step j
  // issues K j+5 and V j+3, and waits for the loads of step j-2.  K 0 and
  // K 1 come first (the prologue's scores), then K 2 (the first fragments
  // read ahead), V 0, K 3, V 1, V 2; K 4 goes into K 0's stage once every
  // wave has read K 0.  Every step issues 2*NLD loads, past the keys
  // included, so each wait has a fixed count.
  issue_k(0, kbuf(0));
  issue_k(1, kbuf(1));
  issue_k(2, kbuf(2));
  issue_v(0, vbuf(0));
  issue_k(3, kbuf(3));
  issue_v(1, vbuf(1));
  issue_v(2, vbuf(2));
#pragma unroll
  for (int ks = 0; ks < DK; ++ks) qf[ks] = qi < p.Sq ? (qf[ks] ^ p.qsign) : u32x4{0u, 0u, 0u, 0u};

  // ---- per-lane fragment read offsets (bytes within a tile)
  // K (A operand of S^T): row 32*kb + n, logical chunk 2*ks + h.
  int koff[DK];
#pragma unroll
  for (int ks = 0; ks < DK; ++ks) koff[ks] = grp * GOFF + n * ROWB + (((2 * ks + h) ^ ksw<D>(n)) << 4);
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
    voff[db] = grp * GOFF + vrow * ROWB + ((chunk ^ vsw<D>(vrow)) << 4) + ((s & 1) << 3);
  }

  // ---- running state of this lane's query
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  // The scores in registers are relative to a per-row reference m_ref (in
  // raw score units): every score product starts from negm = -m_ref in all
  // 16 accumulator slots instead of from 0, so the subtraction costs no
  // instruction.
  float m_ref = 0.f;
  // Running normaliser of this lane's query (both halves hold it): the sum
  // of the rounded P, which divides O.  lse takes l_run + l_corr, where
  // l_corr collects the rounding (unrounded minus rounded P) of the tiles
  // that the vector unit sums: the first tile, the masked tiles and the
  // re-referenced ones.  A short causal row lies wholly in such tiles, so
  // its lse is that of the unrounded P (bf16 rounds P by up to 2^-9, which
  // would otherwise reach ~1e-3 in the lse of a row of a few keys); over the
  // branch-free tiles the rounding errors of many keys average out.
  float l_run = 0.f;
  float l_corr = 0.f;
  const float c = p.c;      // raw score -> exp2 units
  f32x16 negm;
  auto set_negm = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 16; ++r) negm[r] = -m_ref;
  };

  // i-th score product of a tile: S^T[32kb.., q] += K[32kb + n][16ks + 8h ..] q[..]
  auto k_frag = [&](const char* kt, int i) __attribute__((always_inline)) { return lds_read_b128(kt, koff[i % DK] + (i / DK) * 32 * ROWB); };
  // V^T fragment of the P.V product (16-key slice u, d block db)
  auto v_frag = [&](const char* vt, int u, int db) __attribute__((always_inline)) {
    const char* vp = vt + voff[db] + 16 * u * ROWB;
    const u32x2 lo = lds_read_tr16(vp);
    const u32x2 hi = lds_read_tr16(vp + 8 * ROWB);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };
  // scores of the K tile at kt relative to the reference: each 32-key block
  // is a chain of DK products starting from negm
  auto score_tile = [&](f32x16* sacc, const char* kt) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NS; ++i)
      sacc[i / DK] = mfma_32x32x16<BF16>(k_frag(kt, i), qf[i % DK], i % DK == 0 ? negm : sacc[i / DK]);
  };

  // Scores past the keys or (causal) above the diagonal become -inf.
  // sacc[kb][r] = score(qi, k0 + 32kb + 8(r/4) + 4h + r%4).
  // One compare per score: key k0 + 4h + c (c = 32kb + 8(r/4) + r%4, a
  // constant) is masked when c > min(Skl - 1, qir) - k0 - 4h.
  auto apply_mask = [&](f32x16* sacc, int k0) __attribute__((always_inline)) {
    const int lim = (CAUSAL ? min(Skl - 1, qir) : Skl - 1) - k0 - 4 * h;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kb * 32 + 8 * (r >> 2) + (r & 3) > lim) sacc[kb][r] = -INFINITY;
  };

  // Row maximum of a tile's scores (this lane's query, both halves of the
  // wave), in two independent chains of v_maximum3.
  auto tile_max = [&](const f32x16* sacc) __attribute__((always_inline)) -> float {
    float m2[2] = {sacc[0][0], sacc[0][1]};
#pragma unroll
    for (int i = 2; i < 16 * KB; i += 2)
      m2[(i >> 1) & 1] = max3(m2[(i >> 1) & 1], sacc[i >> 4][i & 15], sacc[i >> 4][(i & 15) + 1]);
    return max_halves(__builtin_elementwise_maximum(m2[0], m2[1]));
  };

  auto scale_o = [&](float alpha) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
  };

  // P = exp2(s*c) of the relative scores, packed to 16 bits into pout (a
  // masked score, -inf, gives exp2(-inf) = 0: c > 0 always, see fa_fwd's
  // set-up); returns this lane's sums, in fp32, of the tile's P as rounded to 16 bits
  // (r) and of the rounding, unrounded minus rounded (d), over half of the
  // tile's keys (sum_halves gives the row's).  The branch-free steps ignore
  // them and take the rounded sums on the matrix unit (tile_sum).
  struct Sums {
    float r, d;
  };
  auto tile_exp = [&](const f32x16* sacc, u32x4* pout) __attribute__((always_inline)) -> Sums {
    float ps[2], pu[2];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      float pv[8];
#pragma unroll
      for (int t8 = 0; t8 < 8; ++t8) {
        const float sv = sacc[u >> 1][8 * (u & 1) + t8];
        pv[t8] = __builtin_amdgcn_exp2f(sv * c);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pout[u][e] = pack2<BF16>(pv[2 * e], pv[2 * e + 1]);
        const float pair = sum_pair<BF16>(pout[u][e]);
        const float upair = pv[2 * e] + pv[2 * e + 1];
        ps[e & 1] = (u == 0 && e < 2) ? pair : ps[e & 1] + pair;
        pu[e & 1] = (u == 0 && e < 2) ? upair : pu[e & 1] + upair;
      }
    }
    const float r = ps[0] + ps[1];
    return Sums{r, (pu[0] + pu[1]) - r};
  };

  // Row sums of a tile's packed P on the matrix unit: four 16x16x32
  // products with a constant 0/1 A operand.  Read as a 16x16x32 B operand,
  // the P registers of lane l hold column l%16 and k rows 8(l/16)..+7, that
  // is 8 keys of query l%16 (l/16 even) or of query l%16+16 (l/16 odd),
  // lanes l and l+32 covering the 16 keys of a slice.  A row m of ones over
  // the k blocks of one query puts that query's sum in output row m; rows
  // 0, 8 take queries 0..15 and rows 4, 12 queries 16..31, and output
  // register 0 of lane l is row 4(l/16) of column l%16: the sum of the
  // lane's own query, in both halves of the wave.  Every other output row
  // is zero.  A row's sum also multiplies the other query of its column by
  // zero, so an inf or NaN P of that query makes it NaN; the steps treat a
  // NaN sum like one above the bound and take the rows' sums again, in
  // fp32 on the vector unit.
  const u32x4 ones = [&]() {
    const uint32_t one2 = BF16 ? 0x3f803f80u : 0x3c003c00u;
    const int m = lane & 15, gk = lane >> 4;
    const uint32_t x = ((m & 3) == 0 && ((m >> 2) & 1) == (gk & 1)) ? one2 : 0u;
    return u32x4{x, x, x, x};
  }();
  auto tile_sum = [&](const u32x4* pt) __attribute__((always_inline)) -> float {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < NU; ++u) acc = mfma_16x16x32<BF16>(ones, pt[u], acc);
    return acc[0];
  };

  // The reference moves up to the row's running maximum when some lane's
  // sum over a tile exceeded kSumBound (then its P are no longer known to be
  // small).  st: that tile's scores, exponentiated again into pout; snx: the
  // next tile's scores, formed against the old reference.  O (which holds
  // the products of the earlier tiles) and the running sum are rescaled.
  // Masked scores are -inf already.
  auto reref = [&](f32x16* st, u32x4* pout, f32x16* snx) __attribute__((always_inline)) {
    const float delta = fmaxf(tile_max(st), 0.f);
    m_ref += delta;
    set_negm();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        st[kb][r] -= delta;
        snx[kb][r] -= delta;
      }
    const float alpha = exp2f(-delta * c);
    scale_o(alpha);
    const Sums ts = tile_exp(st, pout);
    l_run = l_run * alpha + sum_halves(ts.r);
    l_corr = l_corr * alpha + sum_halves(ts.d);
  };
  // set by a step whose exponentials hit the bound: the next step, before
  // its products, re-references that tile (its scores are still in the
  // buffer the next step fills with new scores, and its P is the next
  // step's pcur)
  bool redo = false;

  // One step j of the pipeline, with K tile j+2 at kt and V tile j at vt:
  //   matrix unit: scores of tile j+2 (into snext), and O^T += V^T P^T with
  //                P of tile j (pcur, exponentiated by the previous step);
  //   vector unit: exponentials of tile j+1 (scores in scur, formed by the
  //                previous step) into pnext, against the current reference.
  // The two streams share no data, so the interleaved instructions never
  // wait on each other; no row maximum is needed unless a tile's P grows
  // too large (then the next step re-references it first).
  // K fragments read one step ahead by the branch-free steps
  constexpr int NPF = NS;
  u32x4 kpre[NPF];
  auto step_fast = [&](int j, auto jm4_tag, f32x16* scur, f32x16* snext, u32x4* pcur,
                       u32x4* pnext) __attribute__((always_inline)) {
    constexpr int jm = decltype(jm4_tag)::value;  // j % 4
    // The wait and the barrier in one asm statement with a memory clobber:
    // no LDS access moves across it, and no release fence makes the compiler
    // wait for the loads still in flight (they target other stages).  The
    // loads of the previous step may stay in flight; those of step j-2 (K
    // tile j+3, read at the end of this step for the next one, and V tile
    // j+1) have landed.  LDS reads need not have returned: the stages this
    // step overwrites (K tile j+1, whose fragments were read at the end of
    // step j-2, and V tile j-1, read in step j-1) were consumed by the
    // products of the previous step, before this barrier.
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * NLD) : "memory");
    __builtin_amdgcn_sched_barrier(0);
    // the step's products and exponentials run at raised issue priority;
    // the row-sum check and the wait at the next barrier run at the normal
    // one, so a SIMD's other wave, in the middle of its step, issues first
    // (measured: +0.5%)
    __builtin_amdgcn_s_setprio(1);
    // D = 128: the step's loads go between its products (below), so that
    // the waves of a CU do not all fill the address unit's queue at once
    // after the barrier (measured: +1-2% at D = 128, -0.3% at D = 64)
    constexpr int NLS = 2 * NLD;  // loads per step
    constexpr int NMF = NS + NU * DB + NU;  // matrix instructions per step
    constexpr int LSP = D == 128 ? (NMF / NLS >= 4 ? 4 : NMF / NLS) : 0;  // products per load
    if constexpr (LSP == 0) {
      issue_k(j + 5, kbuf((jm + 1) & 3));
      issue_v(j + 3, vbuf((jm + 3) & 3));
    }
    const char* kt = krd((jm + 2) & 3);
    const char* vt = vrd(jm);

    if (redo) reref(snext, pcur, scur);  // (snext still holds the scores of tile j)
    if constexpr (LSP != 0) {
      issue_k(j + 5, kbuf((jm + 1) & 3));
      issue_v(j + 3, vbuf((jm + 3) & 3));
    }
    tile_exp(scur, pnext);
    // the first NPF K fragments of tile j+2 were read by the previous step
#pragma unroll
    for (int i = 0; i < NS; ++i)
      snext[i / DK] = mfma_32x32x16<BF16>(i < NPF ? kpre[i] : k_frag(kt, i), qf[i % DK],
                                          i % DK == 0 ? negm : snext[i / DK]);
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] = mfma_32x32x16<BF16>(v_frag(vt, u, db), pcur[u], oacc[db]);
    const float ts = tile_sum(pnext);
    {
      // one matrix instruction, then up to three (D=64) or two (D=128)
      // vector instructions and two LDS reads (the first K fragments are read up front); the vector
      // work (per 16-key slice 8 multiplies, 8 exponentials and 4 packs)
      // is spread over most of the step
      constexpr int VPM = D == 64 ? 3 : 2;
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
#pragma unroll
      for (int i = 0; i < NMF; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedValu, VPM, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
        if constexpr (LSP != 0)
          if (i % LSP == LSP - 1 && i / LSP < NLS) __builtin_amdgcn_sched_group_barrier(kSchedVmem, 1, 0);
      }
    }
    // K fragments of tile j+3 for the next step
#pragma unroll
    for (int i = 0; i < NPF; ++i) kpre[i] = k_frag(krd((jm + 3) & 3), i);
    // pin the packed P to this block: the packing would otherwise sink past
    // the next step's redo branch, out of the interleaved schedule
#pragma unroll
    for (int u = 0; u < NU; ++u) asm volatile("" ::"v"(pnext[u]));
    __builtin_amdgcn_s_setprio(0);
    redo = __builtin_amdgcn_ballot_w64(!(ts <= kSumBound)) != 0;
    if (!redo) l_run += ts;
  };

  // Any step: the tiles may need masks, and tile j+1 or j+2 may not exist
  // for this wave.  Its stages are compile-time too (jm = j % 4): with a
  // stage chosen at run time the compiler cannot tell which stage the loads
  // in flight write, and waits for all of them before the step's LDS reads.
  auto step_any = [&](int j, auto jm4_tag, f32x16* scur, f32x16* snext, u32x4* pcur,
                      u32x4* pnext) __attribute__((always_inline)) {
    constexpr int jm = decltype(jm4_tag)::value;  // j % 4
    // the same wait and barrier as a branch-free step (and the same
    // argument): a fence here would also wait for the loads of the previous
    // step, which have had one step to land instead of two
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * NLD) : "memory");
    __builtin_amdgcn_sched_barrier(0);
    issue_k(j + 5, kbuf((jm + 1) & 3));
    issue_v(j + 3, vbuf((jm + 3) & 3));
    if (j < nt_w) {
      const char* kt = krd((jm + 2) & 3);
      const char* vt = vrd(jm);
      if (redo) reref(snext, pcur, scur);
      if (j + 2 < nt_w) score_tile(snext, kt);
      float ts = 0.f, td = 0.f;
      if (j + 1 < nt_w) {
        // tiles before j_mask hold only keys before the end and at or
        // below the wave's first query: no score of theirs is masked
        if (j + 1 >= j_mask) apply_mask(scur, (j + 1) * BN);
        const Sums t2 = tile_exp(scur, pnext);
        ts = sum_halves(t2.r);
        td = sum_halves(t2.d);
      }
#pragma unroll
      for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] = mfma_32x32x16<BF16>(v_frag(vt, u, db), pcur[u], oacc[db]);
      redo = __builtin_amdgcn_ballot_w64(ts > kSumBound) != 0;
      if (!redo) {
        l_run += ts;
        l_corr += td;
      }
    }
  };

  // ---- prologue: scores of tiles 0 and 1, P of tile 0
  f32x16 sa[KB], sb[KB];
  u32x4 pa[NU], pb[NU];
  // K 0, K 1 and K 2 have landed (in every wave: the barrier); the loads
  // after them may stay in flight (no fence)
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(4 * NLD) : "memory");
  __builtin_amdgcn_sched_barrier(0);
  if (nt_w > 0) {
    // tile 0 from a zero reference; its row maximum becomes the reference.
    // Key 0 of the range is masked only for a causal row that sees no key of
    // the range at all (a split with i < kb0): that row keeps a zero
    // reference, its P are all 0 and its sum stays 0.
    set_negm();
    score_tile(sa, krd(0));
    if (j_mask == 0) apply_mask(sa, 0);  // (as in the general steps)
    m_ref = tile_max(sa);
    if ((SPLIT || KG > 1) && CAUSAL && m_ref == -INFINITY) m_ref = 0.f;
    set_negm();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sa[kb][r] -= m_ref;
    const Sums t0 = tile_exp(sa, pa);
    l_run = sum_halves(t0.r);
    l_corr = sum_halves(t0.d);
    score_tile(sb, krd(1));
  }

  // step j: scores of tile j+1 in sb (j even) or sa (j odd), P of tile j in
  // pa (j even) or pb (j odd)
  int j = 0;
  if (j_fast > 0) {
#pragma unroll
    for (int i = 0; i < NPF; ++i) kpre[i] = k_frag(krd(2), i);
  }
  // every wave's reads of K tile 0 were consumed by its prologue products:
  // the stage can take K tile 4
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  issue_k(4, kbuf(0));
  for (; j < j_fast; j += 4) {
    step_fast(j, Int<0>{}, sb, sa, pa, pb);
    step_fast(j + 1, Int<1>{}, sa, sb, pb, pa);
    step_fast(j + 2, Int<2>{}, sb, sa, pa, pb);
    step_fast(j + 3, Int<3>{}, sa, sb, pb, pa);
  }
  // (j is a multiple of 4 here; the conditions are the same for every wave
  // of the work-group, so every wave meets every barrier)
  for (; j < nsteps; j += 4) {
    step_any(j, Int<0>{}, sb, sa, pa, pb);
    if (j + 1 < nsteps) step_any(j + 1, Int<1>{}, sa, sb, pb, pa);
    if (j + 2 < nsteps) step_any(j + 2, Int<2>{}, sb, sa, pa, pb);
    if (j + 3 < nsteps) step_any(j + 3, Int<3>{}, sa, sb, pb, pa);
  }

  // the last steps' loads (past the keys) are still in flight: let them land
  // before the work-group's LDS can be handed to another
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  if constexpr (KG == 2) {
    // Group 1 hands its partial result to group 0 through LDS (the K stages
    // hold O, one wave per stage; the V stages m, l and the rounding
    // correction).  Both partials are against their own reference: with M
    // the larger, each is rescaled by 2^(c (m_g - M)), the online softmax's
    // own rescaling.  A group that saw no key of a row has l = 0 and weighs
    // nothing; a NaN row stays NaN.
    float* ob = reinterpret_cast<float*>(wave == 0 ? kst0 : wave == 1 ? kst1 : wave == 2 ? kst2 : kst3);
    float* mb = reinterpret_cast<float*>(wave == 0 ? vst0 : wave == 1 ? vst1 : wave == 2 ? vst2 : vst3);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // every wave is done with the tiles
    __builtin_amdgcn_sched_barrier(0);
    if (grp == 1) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) ob[(db * 16 + r) * 64 + lane] = oacc[db][r];
      mb[lane] = m_ref;
      mb[64 + lane] = l_run;
      mb[128 + lane] = l_corr;
    }
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if (grp == 1) return;
    const float m1 = mb[lane], l1 = mb[64 + lane], c1 = mb[128 + lane];
    const float mm = l1 == 0.f ? m_ref : __builtin_elementwise_maximum(m_ref, m1);
    const float a0 = exp2f((m_ref - mm) * c);
    const float a1 = l1 == 0.f ? 0.f : exp2f((m1 - mm) * c);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] = oacc[db][r] * a0 + ob[(db * 16 + r) * 64 + lane] * a1;
    l_run = l_run * a0 + l1 * a1;
    l_corr = l_corr * a0 + c1 * a1;
    m_ref = mm;
  }

  // ---- epilogue: normalise, round, store O rows and lse
  if (SPLIT && qi < p.Sq) {
    // the range's partial result, fp32: O normalised over the range's keys
    // and its lse; a row that sees none of them gets 0 and -inf (zero
    // weight in the merge)
    const float l = l_run;
    const size_t row = ((size_t)split * p.n_bh + bh) * p.Sq + qi;
    const float inv = l == 0.f ? 0.f : 1.f / l;
    float* op = p.po + row * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d0 = db * 32 + 8 * gq + 4 * h;
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = oacc[db][4 * gq + e] * inv;
        *reinterpret_cast<f32x4*>(op + d0) = w;
      }
    if (h == 0) p.plse[row] = l == 0.f ? -INFINITY : (m_ref * c + __log2f(l + l_corr)) * kLn2;
  }
  if constexpr (!SPLIT && KG == 1) {
    // O through the LDS, so that it is stored in whole rows (16-byte stores
    // that complete 128-byte lines) rather than 16 bytes into each of 32
    // rows per store: every wave has read all of the stages, and each writes
    // its 32 rows of O into its own K stage, 16-byte chunk cc of row r at
    // cc ^ f(r): the reads (whole rows) are free of bank conflicts, and the
    // writes (32 rows at one chunk) conflict two ways at most, rows r and
    // r + 16 taking the same banks (32-64 conflict cycles per wave measured,
    // well under 1% of the kernel's LDS activity).  Measured: +1-1.4% at
    // D = 128, unchanged at D = 64.
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    char* ob = kbuf(wave);
    auto osw = [](int r) __attribute__((always_inline)) { return D == 64 ? ((r >> 1) & 7) : (r & 15); };
    const float inv = 1.f / l_run;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        u32x2 w;
        w[0] = pack2<BF16>(oacc[db][4 * gq] * inv, oacc[db][4 * gq + 1] * inv);
        w[1] = pack2<BF16>(oacc[db][4 * gq + 2] * inv, oacc[db][4 * gq + 3] * inv);
        const int cc = db * 4 + gq;  // the chunk of d = 32 db + 8 gq + 4 h .. +3
        *reinterpret_cast<u32x2*>(ob + n * ROWB + ((cc ^ osw(n)) << 4) + h * 8) = w;
      }
    if (qi < p.Sq && h == 0) p.lse[(size_t)bh * p.Sq + qi] = (m_ref * c + __log2f(l_run + l_corr)) * kLn2;
    uint16_t* og = p.o + ((size_t)bh * p.Sq + qw0) * D;
#pragma unroll
    for (int i = 0; i < 32 * ROWB / 1024; ++i) {
      const int lin = i * 64 + lane;
      const int r = lin / CH, cc = lin % CH;
      const u32x4 v = *reinterpret_cast<const u32x4*>(ob + r * ROWB + ((cc ^ osw(r)) << 4));
      if (qw0 + r < p.Sq) *reinterpret_cast<u32x4*>(og + r * D + cc * 8) = v;
    }
    return;
  }
  if (!SPLIT && qw0 < p.Sq) {
    const float l = l_run;
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
      if (h == 0) p.lse[(size_t)bh * p.Sq + qi] = (m_ref * c + __log2f(l + l_corr)) * kLn2;
    }
  }
}

// Keys per tile.  At D=128 always 32 (two work-groups per CU).  At D=64, a
// launch that fills the chip takes 32-key tiles with three work-groups per CU
// (measured about 2% faster than 64-key tiles with two); a launch of at most
// kSmallGrid work-groups, which runs as a single wave of work-groups, takes
// 64-key tiles: half the steps per work-group, and its latency is the
// launch's (measured 6% faster on 128 work-groups).  A launch of at most
// kHalfGrid work-groups (no split over the keys) would leave half of the CUs
// idle and last as long as its longest block's work on one CU: it runs with
// two key groups of two waves instead, 64 queries per work-group, so that
// twice as many work-groups each do half of a block's keys.
constexpr int64_t kSmallGrid = 512;
constexpr int64_t kHalfGrid = 128;

template <int D, bool BF16, bool CAUSAL, bool SPLIT>
hipError_t launch(const Params& base, int64_t BH, int64_t Sq, hipStream_t stream) {
  Params p = base;
  p.n_qblk = (int)((Sq + kBM - 1) / kBM);
  p.n_wg = (int)(BH * p.n_qblk * p.n_split);
  const void* fn = reinterpret_cast<const void*>(&fa_fwd_kernel<D, BF16, CAUSAL, 32, SPLIT>);
  if constexpr (D == 64)
    if (p.n_wg <= kSmallGrid) fn = reinterpret_cast<const void*>(&fa_fwd_kernel<D, BF16, CAUSAL, 64, SPLIT>);
  if constexpr (!SPLIT)
    if (p.n_wg <= kHalfGrid) {
      fn = reinterpret_cast<const void*>(&fa_fwd_kernel<D, BF16, CAUSAL, D == 64 ? 64 : 32, SPLIT, 2>);
      p.n_qblk = (int)((Sq + kBM / 2 - 1) / (kBM / 2));
      p.n_wg = (int)(BH * p.n_qblk);
    }
  // Causal blocks run longest first across an XCD's heads (when the heads
  // split evenly over the 8 XCDs): head by head, the long blocks of the
  // XCD's last heads would start late (simulated: 1.21x the balanced time
  // at 32 blocks on 64 slots, measured +9% on B4 H16 S4096 D128).  With more
  // blocks per head than slots it still measured +1.0% (B1 H32 S16384
  // D128, 128 blocks on 64 slots), though fewer heads' keys then share the
  // XCD's L2 at a time in the head-by-head order.
  p.xcd_heads = (CAUSAL && !SPLIT && BH % 8 == 0) ? (int)(BH / 8) : 0;
  void* args[] = {&p};
  return hipLaunchKernel(fn, dim3(p.n_wg), dim3(64 * kWaves), args, 0, stream);
}

template <bool SPLIT>
hipError_t launch_any(const Params& p, int64_t BH, int64_t Sq, int64_t D, bool bf, bool causal, hipStream_t s) {
  if (D == 64) {
    if (bf) return causal ? launch<64, true, true, SPLIT>(p, BH, Sq, s) : launch<64, true, false, SPLIT>(p, BH, Sq, s);
    return causal ? launch<64, false, true, SPLIT>(p, BH, Sq, s) : launch<64, false, false, SPLIT>(p, BH, Sq, s);
  }
  if (bf) return causal ? launch<128, true, true, SPLIT>(p, BH, Sq, s) : launch<128, true, false, SPLIT>(p, BH, Sq, s);
  return causal ? launch<128, false, true, SPLIT>(p, BH, Sq, s) : launch<128, false, false, SPLIT>(p, BH, Sq, s);
}

// Log-sum-exp merge of partial results over disjoint key ranges (the online
// softmax's rescaling to a common maximum, applied to finished partials):
//   M = max_g lse_g,  lse = M + ln sum_g e^(lse_g - M),  o = sum_g e^(lse_g - lse) o_g
// rounded to the storage type.  Parts with lse_g = -inf weigh nothing; a row
// with only such parts gets lse = -inf and o = 0.  D/4 threads per row, 4
// consecutive elements each (16-byte loads of every part).
template <int D, bool BF16>
__global__ __launch_bounds__(256) void lse_merge_kernel(const float* po, const float* plse, int n_part,
                                                       int64_t rows, uint16_t* o, float* lse) {
  constexpr int TPR = D / 4;
  constexpr int RPB = 256 / TPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int d0 = (threadIdx.x % TPR) * 4;
  if (row >= rows) return;
  float M = -INFINITY;
  for (int g = 0; g < n_part; ++g) M = __builtin_elementwise_maximum(M, plse[(int64_t)g * rows + row]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float L = -INFINITY;
  if (M != -INFINITY) {
    float sum = 0.f;
    for (int g = 0; g < n_part; ++g) sum += expf(plse[(int64_t)g * rows + row] - M);
    L = M + logf(sum);
    for (int g = 0; g < n_part; ++g) {
      const float w = expf(plse[(int64_t)g * rows + row] - L);
      const f32x4 x = *reinterpret_cast<const f32x4*>(po + ((int64_t)g * rows + row) * D + d0);
      acc += w * x;
    }
  }
  u32x2 out;
  out[0] = pack2<BF16>(acc[0], acc[1]);
  out[1] = pack2<BF16>(acc[2], acc[3]);
  *reinterpret_cast<u32x2*>(o + row * D + d0) = out;
  if (d0 == 0) lse[row] = L;
}

hipError_t launch_merge(const float* po, const float* plse, int64_t n_part, int64_t rows, int64_t D, bool bf,
                        void* o, float* lse, hipStream_t s) {
  const int rpb = (int)(256 / (D / 4));
  const int64_t blocks = (rows + rpb - 1) / rpb;
  uint16_t* ob = static_cast<uint16_t*>(o);
  const int np = (int)n_part;
  if (D == 64) {
    if (bf) lse_merge_kernel<64, true><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(po, plse, np, rows, ob, lse);
    else lse_merge_kernel<64, false><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(po, plse, np, rows, ob, lse);
  } else {
    if (bf) lse_merge_kernel<128, true><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(po, plse, np, rows, ob, lse);
    else lse_merge_kernel<128, false><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(po, plse, np, rows, ob, lse);
  }
  return hipGetLastError();
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// Host-side checks shared by the entry points: pointers, sizes, index
// ranges and overlaps of the attention arguments (no device access).
fa_status check_attention_args(const void* q, const void* k, const void* v, const void* o, const float* lse,
                               int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D, float scale,
                               int dtype) {
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
  if (BH >= lim / ((Sq + kBM - 1) / kBM)) return FA_ERR_INVALID_ARG;
  // element counts in int64: BH < 2^31 and S*D < 2^31 keep these below 2^62
  const size_t qo_bytes = (size_t)(BH * Sq * D) * 2, kv_bytes = (size_t)(BH * Sk * D) * 2;
  const size_t lse_bytes = (size_t)(BH * Sq) * 4;
  if (overlaps(o, qo_bytes, q, qo_bytes) || overlaps(o, qo_bytes, k, kv_bytes) ||
      overlaps(o, qo_bytes, v, kv_bytes) || overlaps(lse, lse_bytes, q, qo_bytes) ||
      overlaps(lse, lse_bytes, k, kv_bytes) || overlaps(lse, lse_bytes, v, kv_bytes) ||
      overlaps(o, qo_bytes, lse, lse_bytes))
    return FA_ERR_INVALID_ARG;
  return FA_OK;
}

Params make_params(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                   int64_t Sq, int64_t Sk, float scale) {
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
  // scores times c are the exponents of 2; c is at least 1e-30 so that a
  // masked score (-inf) gives exp2(-inf) = 0 with no test in the kernel, also
  // for scale 0 (where -inf * 0 would be NaN).  With scale 0 every other
  // exponent is then below 2^-60 in size for any finite score under 2^39,
  // and exp2 returns exactly 1, as for c = 0.
  p.c = (float)fmax(fabs((double)scale) * 1.4426950408889634, 1e-30);
  p.qsign = scale < 0.f ? 0x80008000u : 0u;
  p.n_split = 1;
  p.kchunk = (int)Sk;
  p.n_bh = (int)(B * H);
  p.po = nullptr;
  p.plse = nullptr;
  return p;
}

// Key ranges of a split: the requested count (or, for 0, enough ranges to
// give about kAutoSplitBlocks work-groups, with at least 256 keys each),
// at least 64 keys per range; ranges are a multiple of 64 keys long, so the
// count actually used may be smaller than the one asked for.
constexpr int64_t kAutoSplitBlocks = 2048;
struct SplitPlan {
  int64_t n, chunk;
};
SplitPlan split_plan(int64_t BH, int64_t Sq, int64_t Sk, int64_t n_split) {
  const int64_t wgs = BH * ((Sq + kBM - 1) / kBM);
  int64_t n = n_split;
  if (n <= 0) n = min((kAutoSplitBlocks + wgs - 1) / wgs, max((int64_t)1, Sk / 256));
  n = max((int64_t)1, min(n, (Sk + 63) / 64));
  const int64_t chunk = ((Sk + n - 1) / n + 63) / 64 * 64;
  return {(Sk + chunk - 1) / chunk, chunk};
}

}  // namespace

extern "C" fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                            int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                            float scale, int causal, int dtype, void* stream) {
  const fa_status st = check_attention_args(q, k, v, o, lse, B, H, Sq, Sk, D, scale, dtype);
  if (st != FA_OK) return st;
  const Params p = make_params(q, k, v, o, lse, B, H, Sq, Sk, scale);
  const hipError_t err =
      launch_any<false>(p, B * H, Sq, D, dtype == FA_BF16, causal != 0, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

extern "C" int64_t fa_fwd_split_count(int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t n_split) {
  if (B < 1 || H < 1 || Sq < 1 || Sk < 1 || n_split < 0) return 0;
  return split_plan(B * H, Sq, Sk, n_split).n;
}

extern "C" size_t fa_fwd_split_workspace_size(int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                                              int64_t n_split) {
  if (B < 1 || H < 1 || Sq < 1 || Sk < 1 || D < 1 || n_split < 0) return 0;
  const int64_t lim = (int64_t)1 << 31;
  if (B >= lim || H >= lim || Sq >= lim || Sk >= lim || D > 1024 || B * H >= lim / ((Sq + kBM - 1) / kBM)) return 0;
  const int64_t n = split_plan(B * H, Sq, Sk, n_split).n;
  // n * B*H*Sq < 2^31 * 128 rows (the grid limit of fa_fwd_split), times (D+1)*4 bytes
  if (B * H * ((Sq + kBM - 1) / kBM) >= lim / n) return 0;
  return (size_t)n * (size_t)(B * H * Sq) * (size_t)(D + 1) * 4u;
}

namespace {

// The key split with its partials in `workspace` (a caller buffer or the
// fixed scratch): argument checks, the partial-result kernel, the merge.
fa_status split_impl(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                     int64_t Sq, int64_t Sk, int64_t D, float scale, int causal, int dtype, int64_t n_split,
                     void* workspace, size_t workspace_bytes, void* stream) {
  fa_status st = check_attention_args(q, k, v, o, lse, B, H, Sq, Sk, D, scale, dtype);
  if (st != FA_OK) return st;
  if (n_split < 0 || !workspace || ((uintptr_t)workspace & 15u)) return FA_ERR_INVALID_ARG;
  const int64_t BH = B * H;
  const SplitPlan sp = split_plan(BH, Sq, Sk, n_split);
  const int64_t lim = (int64_t)1 << 31;
  if (BH * ((Sq + kBM - 1) / kBM) >= lim / sp.n) return FA_ERR_INVALID_ARG;
  if ((BH * Sq + 15) / 16 >= lim) return FA_ERR_INVALID_ARG;  // the merge's grid
  const size_t need = fa_fwd_split_workspace_size(B, H, Sq, Sk, D, n_split);
  if (workspace_bytes < need) return FA_ERR_INVALID_ARG;
  const size_t qo_bytes = (size_t)(BH * Sq * D) * 2, kv_bytes = (size_t)(BH * Sk * D) * 2;
  const size_t lse_bytes = (size_t)(BH * Sq) * 4;
  if (overlaps(workspace, need, q, qo_bytes) || overlaps(workspace, need, k, kv_bytes) ||
      overlaps(workspace, need, v, kv_bytes) || overlaps(workspace, need, o, qo_bytes) ||
      overlaps(workspace, need, lse, lse_bytes))
    return FA_ERR_INVALID_ARG;

  Params p = make_params(q, k, v, o, lse, B, H, Sq, Sk, scale);
  p.n_split = (int)sp.n;
  p.kchunk = (int)sp.chunk;
  p.po = static_cast<float*>(workspace);
  p.plse = p.po + (size_t)sp.n * (size_t)(BH * Sq) * (size_t)D;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf = dtype == FA_BF16;
  if (launch_any<true>(p, BH, Sq, D, bf, causal != 0, s) != hipSuccess) return FA_ERR_LAUNCH;
  if (launch_merge(p.po, p.plse, sp.n, BH * Sq, D, bf, o, lse, s) != hipSuccess) return FA_ERR_LAUNCH;
  return FA_OK;
}

// Device address of `scratch` on the current device, looked up on the first
// call made with that device current and kept: every device has its own copy
// of the array at its own address.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

fa_status scratch_on_current_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FA_ERR_LAUNCH;
  if (dev >= kMaxDevices) return FA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FA_ERR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return FA_OK;
}

}  // namespace

extern "C" fa_status fa_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                                  int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                                  float scale, int causal, int dtype, int64_t n_split,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  return split_impl(q, k, v, o, lse, B, H, Sq, Sk, D, scale, causal, dtype, n_split, workspace,
                    workspace_bytes, stream);
}

extern "C" fa_status fa_fwd_split_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                          int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                                          float scale, int causal, int dtype, int64_t n_split, void* stream) {
  // the same checks as fa_fwd_split first, so that a bad argument is
  // reported as such and not as a size beyond the scratch
  fa_status st = check_attention_args(q, k, v, o, lse, B, H, Sq, Sk, D, scale, dtype);
  if (st != FA_OK) return st;
  if (n_split < 0) return FA_ERR_INVALID_ARG;
  const size_t need = fa_fwd_split_workspace_size(B, H, Sq, Sk, D, n_split);
  if (need == 0) return FA_ERR_INVALID_ARG;
  if (need > (size_t)FA_SPLIT_SCRATCH_BYTES) return FA_ERR_SCRATCH_TOO_SMALL;
  void* ws = nullptr;
  st = scratch_on_current_device(&ws);
  if (st != FA_OK) return st;
  return split_impl(q, k, v, o, lse, B, H, Sq, Sk, D, scale, causal, dtype, n_split, ws,
                    (size_t)FA_SPLIT_SCRATCH_BYTES, stream);
}

extern "C" fa_status fa_lse_merge(const float* o_parts, const float* lse_parts, int64_t n_part, int64_t rows,
                                  int64_t D, void* o, float* lse, int dtype, void* stream) {
  if (!o_parts || !lse_parts || !o || !lse) return FA_ERR_INVALID_ARG;
  if ((((uintptr_t)o_parts | (uintptr_t)o) & 15u) || (((uintptr_t)lse_parts | (uintptr_t)lse) & 3u))
    return FA_ERR_INVALID_ARG;
  if (n_part < 1 || rows < 1 || D < 1) return FA_ERR_INVALID_ARG;
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
  const int64_t lim = (int64_t)1 << 31;
  if (n_part >= lim || rows >= ((int64_t)1 << 40) / D || n_part >= ((int64_t)1 << 52) / (rows * D))
    return FA_ERR_INVALID_ARG;
  if ((rows + 255) / (256 / (D / 4)) >= lim) return FA_ERR_INVALID_ARG;
  const size_t po_bytes = (size_t)(n_part * rows * D) * 4, pl_bytes = (size_t)(n_part * rows) * 4;
  const size_t o_bytes = (size_t)(rows * D) * 2, l_bytes = (size_t)rows * 4;
  if (overlaps(o, o_bytes, o_parts, po_bytes) || overlaps(o, o_bytes, lse_parts, pl_bytes) ||
      overlaps(lse, l_bytes, o_parts, po_bytes) || overlaps(lse, l_bytes, lse_parts, pl_bytes) ||
      overlaps(o, o_bytes, lse, l_bytes))
    return FA_ERR_INVALID_ARG;
  const hipError_t err =
      launch_merge(o_parts, lse_parts, n_part, rows, D, dtype == FA_BF16, o, lse, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

extern "C" const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARG: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported head dimension or dtype";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_SCRATCH_TOO_SMALL: return "partial results exceed the library's fixed scratch buffer";
    default: return "unknown status";
  }
}
