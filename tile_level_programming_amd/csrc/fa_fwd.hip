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
// CDNA4 mapping (one work-group = one (batch, head, block of BM queries)):
//
//  * Each wave owns 32 queries.  Scores are formed transposed, S^T = K Q^T,
//    with v_mfma_f32_32x32x16_{f16,bf16}: K (from LDS) is the A operand and
//    the wave's Q fragment (kept in VGPRs for the whole loop) is the B
//    operand.  In the 32x32 accumulator layout a lane holds one column (one
//    query) and 16 rows (keys), so each lane owns a query: the row maximum and
//    sum are in-lane, plus one exchange with the lane 32 away for the max.
//  * O is accumulated transposed as well, O^T = V^T P^T: the exponentiated
//    scores, packed to 16 bits in registers, are directly the B operand (the
//    lane layout of a B operand equals the accumulator's column ownership),
//    and V^T comes from LDS.  The order in which a product's K slots visit the
//    keys is free; the V^T tile is stored with the matching key permutation so
//    that each lane's A fragment is one 16-byte LDS read.
//  * The rescale factor alpha is per query, i.e. per lane: rescaling O is a
//    plain per-lane multiply.
//  * exp is exp2 with scale*log2(e) folded into one FMA per score.
//  * K and V tiles of BN keys are double-buffered in LDS; the global loads of
//    tile j+1 (128-bit, coalesced) are in flight while tile j is computed.
//  * Causal: key tiles past the block's last query are never loaded; a wave
//    skips the products of tiles that lie wholly above its queries; only tiles
//    that cross the diagonal (or the end of the keys) are masked.
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

constexpr float kLn2 = 0.6931471805599453f;

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

__device__ __forceinline__ float xchg32(float x) {
  // value held by the lane 32 away (the other half of the wave)
  return __shfl_xor(x, 32, 64);
}

// Key position inside the LDS V^T row: swap bits 2 and 3 of the key index, so
// that the 8 keys one lane feeds to one P.V product slot range are adjacent.
__device__ __forceinline__ int vt_pos(int key) {
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
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

template <int D, bool BF16, bool CAUSAL, int NW, int BN>
__global__ __launch_bounds__(NW * 64) void fa_fwd_kernel(Params p) {
  constexpr int NT = NW * 64;        // threads per work-group
  constexpr int BM = NW * 32;        // queries per work-group
  constexpr int KS = D + 8;          // LDS row stride of the K tile (halves), padded
  constexpr int VS = BN + 8;         // LDS row stride of the V^T tile (halves), padded
  constexpr int STAGE = BN * KS + D * VS;
  constexpr int CH = D / 8;          // 16-byte chunks per row
  constexpr int NCH = BN * CH / NT;  // chunks per thread per tile and tensor
  constexpr int KB = BN / 32;        // 32-key blocks per tile
  constexpr int NU = BN / 16;        // 16-key slices per tile (P.V product steps)
  constexpr int DK = D / 16;         // k-steps of the score product
  constexpr int DB = D / 32;         // 32-wide d blocks of the output
  static_assert(BN % 32 == 0 && (BN * CH) % NT == 0, "tile shape");

  __shared__ u32x4 lds_raw[(2 * STAGE * 2 + 15) / 16];
  uint16_t* lds = reinterpret_cast<uint16_t*>(lds_raw);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 31;   // query column owned by this lane
  const int h = lane >> 5;   // which half of the wave

  const int t = xcd_remap(blockIdx.x, p.n_wg);
  const int bh = t / p.n_qblk;
  int qb = t - bh * p.n_qblk;
  if (CAUSAL) qb = p.n_qblk - 1 - qb;  // longest blocks first
  const int q0 = qb * BM;
  const int qw0 = q0 + wave * 32;     // first query of this wave
  const int qi = qw0 + n;             // query of this lane

  const uint16_t* qg = p.q + (size_t)bh * p.Sq * D;
  const uint16_t* kg = p.k + (size_t)bh * p.Sk * D;
  const uint16_t* vg = p.v + (size_t)bh * p.Sk * D;

  // ---- Q fragment: B operand of S^T = K Q^T, lane holds q[qi][16*ks + 8*h .. +8]
  u32x4 qf[DK];
#pragma unroll
  for (int ks = 0; ks < DK; ++ks) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (qi < p.Sq) x = *reinterpret_cast<const u32x4*>(qg + (size_t)qi * D + ks * 16 + h * 8);
    x ^= p.qsign;
    qf[ks] = x;
  }

  const int kend = CAUSAL ? min(p.Sk, q0 + BM) : p.Sk;
  const int ntiles = (kend + BN - 1) / BN;

  // ---- global -> register staging of one K and V tile
  u32x4 kr[NCH], vr[NCH];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int cidx = tid + i * NT;
      const int row = cidx / CH, col = cidx % CH;
      const int key = k0 + row;
      u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
      if (key < p.Sk) {
        a = *reinterpret_cast<const u32x4*>(kg + (size_t)key * D + col * 8);
        b = *reinterpret_cast<const u32x4*>(vg + (size_t)key * D + col * 8);
      }
      kr[i] = a;
      vr[i] = b;
    }
  };
  auto sstore = [&](int buf) {
    uint16_t* ks_ = lds + buf * STAGE;
    uint16_t* vt_ = ks_ + BN * KS;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int cidx = tid + i * NT;
      const int row = cidx / CH, col = cidx % CH;
      *reinterpret_cast<u32x4*>(ks_ + row * KS + col * 8) = kr[i];
      const int pos = vt_pos(row);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w = vr[i][e];
        vt_[(col * 8 + 2 * e) * VS + pos] = (uint16_t)(w & 0xFFFFu);
        vt_[(col * 8 + 2 * e + 1) * VS + pos] = (uint16_t)(w >> 16);
      }
    }
  };

  // ---- running state of this lane's query
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_run = -INFINITY;  // running max of the raw (unscaled) scores
  float l_run = 0.f;        // this half's share of the running normaliser
  const float c = p.c;

  gload(0);
  sstore(0);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int k0 = j * BN;
    if (j + 1 < ntiles) gload(k0 + BN);

    const bool active = !CAUSAL || k0 <= qw0 + 31;  // some key of the tile is visible to the wave
    if (active && qw0 < p.Sq) {
      const uint16_t* ks_ = lds + (j & 1) * STAGE;
      const uint16_t* vt_ = ks_ + BN * KS;

      // S^T = K Q^T for the tile: s[kb][r] = score(query qi, key k0 + 32kb + 8(r/4) + 4h + r%4)
      f32x16 s[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < DK; ++ks) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(ks_ + (kb * 32 + n) * KS + ks * 16 + h * 8);
          s[kb] = mfma_32x32x16<BF16>(a, qf[ks], s[kb]);
        }
      }

      const bool masked = (k0 + BN > p.Sk) || (CAUSAL && k0 + BN - 1 > qw0);
      if (masked) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            const bool hide = key >= p.Sk || (CAUSAL && key > qi);
            if (hide) s[kb][r] = -INFINITY;
          }
      }

      // online softmax: new running max, rescale factor, probabilities
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = fmaxf(mx, xchg32(mx));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = (m_run == -INFINITY) ? 0.f : exp2f((m_run - m_new) * c);
      const float mc = m_new * c;
      m_run = m_new;

      float psum = 0.f;
      u32x4 pf[NU];
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        float pv[8];
#pragma unroll
        for (int t8 = 0; t8 < 8; ++t8) {
          const float sv = s[u >> 1][8 * (u & 1) + t8];
          float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(sv, c, -mc));
          if (masked && sv == -INFINITY) pe = 0.f;
          pv[t8] = pe;
          psum += pe;
        }
        pf[u][0] = pack2<BF16>(pv[0], pv[1]);
        pf[u][1] = pack2<BF16>(pv[2], pv[3]);
        pf[u][2] = pack2<BF16>(pv[4], pv[5]);
        pf[u][3] = pack2<BF16>(pv[6], pv[7]);
      }
      l_run = alpha * l_run + psum;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;

      // O^T += V^T P^T
#pragma unroll
      for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(vt_ + (db * 32 + n) * VS + u * 16 + h * 8);
          oacc[db] = mfma_32x32x16<BF16>(a, pf[u], oacc[db]);
        }
    }

    if (j + 1 < ntiles) sstore((j + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: normalise, round, store O rows and lse
  if (qi < p.Sq) {
    const float l = l_run + xchg32(l_run);
    const float inv = 1.f / l;
    uint16_t* og = p.o + ((size_t)bh * p.Sq + qi) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = db * 32 + 8 * g + 4 * h;
        u32x2 w;
        w[0] = pack2<BF16>(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv);
        w[1] = pack2<BF16>(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
        *reinterpret_cast<u32x2*>(og + d0) = w;
      }
    if (h == 0) p.lse[(size_t)bh * p.Sq + qi] = (m_run * c + __log2f(l)) * kLn2;
  }
}

template <int D, bool BF16, bool CAUSAL>
struct Cfg {
  static constexpr int NW = 4;
  static constexpr int BN = 64;
};

template <int D, bool BF16, bool CAUSAL>
hipError_t launch(const Params& base, int64_t BH, int64_t Sq, hipStream_t stream) {
  using C = Cfg<D, BF16, CAUSAL>;
  constexpr int BM = C::NW * 32;
  Params p = base;
  p.n_qblk = (int)((Sq + BM - 1) / BM);
  p.n_wg = (int)(BH * p.n_qblk);
  void* args[] = {&p};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fa_fwd_kernel<D, BF16, CAUSAL, C::NW, C::BN>),
                         dim3(p.n_wg), dim3(C::NW * 64), args, 0, stream);
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
  const int64_t minBM = 128;
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
