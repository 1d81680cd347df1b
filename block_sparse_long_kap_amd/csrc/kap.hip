// Kernel-Aware Proxy (KAP) for gfx950: block-pooled scoring, "have rowmax"
// flags, flag-grouped ordering and stage-1 budget truncation.
//
// Method: CoSA (paper text on paperpeel.com), §4.2 "Kernel-Aware Proxy
// Design" with App. C.1 "Illustrative KAP Ordering": every candidate key
// block of a query block receives an importance score and an HRM flag; the
// HRM and non-HRM groups are sorted independently by score, the HRM group is
// placed first and the leading entries under the stage-1 budget form the
// ordered mask M_KAP.  §5.1 ("Implementation details") fuses scoring and
// pooling to keep the proxy cheap.  The body of "Block ranking" is not in
// the text; the score used here is the block-pooled logit (mean query of 16
// consecutive rows against the mean key of a page), its per-proxy-row softmax
// averaged over the tile's proxy rows, and HRM marks the arg-max block of
// each proxy row.
//
// Two launches:
//   kap_pool_keys  one workgroup per (sequence, key block, KV head): streams
//                  the head's page once from HBM and writes the fp32 mean key
//                  split into bf16 hi + lo halves (x ~= hi + lo to 16 bits).
//   kap_select     one workgroup per (sequence, query head, 4 consecutive
//                  tiles): pools the tiles' queries from HBM (4 x 8 proxy rows
//                  = one 32-row MFMA operand), scores every candidate block
//                  with v_mfma_f32_32x32x16_bf16 on the split operands
//                  (hi*hi + hi*lo + lo*hi, fp32-level accuracy), takes
//                  per-row max / arg-max / sum online in a first pass,
//                  recomputes the scores for the weights in a second pass,
//                  builds 64-bit keys (not HRM, -w, j) in LDS, radix-selects
//                  the k smallest per tile and bitonic-sorts only those (one
//                  wavefront per tile, no workgroup barrier), and writes the
//                  first k ids of each tile with their remapped pages.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cosa_internal.h"

namespace cosa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kTilesPerGroup = 4;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// x ~= hi + lo with hi = bf16(x) and lo = bf16(x - hi)
__device__ __forceinline__ void split_bf16(float x, uint16_t& hi, uint16_t& lo) {
  const __bf16 h = (__bf16)x;
  const __bf16 l = (__bf16)(x - (float)h);
  hi = __builtin_bit_cast(uint16_t, h);
  lo = __builtin_bit_cast(uint16_t, l);
}

// ---------------------------------------------------------------------------
// Key pooling: the mean of the valid keys of block j, plane 0 = bf16 hi,
// plane 1 = bf16 lo, stored for the score product's operand reads: element d
// of block j at [(j / 32)][d / 16][(d / 8) % 2][j % 32][d % 8] of its
// (plane, sequence, KV head) slab, so that one k-step of 32 blocks is 1 KB of
// consecutive bytes (one coalesced 16-byte read per lane).
template <int D>
__device__ __forceinline__ int64_t kbar_offset(int j, int d) {
  return ((((int64_t)(j >> 5) * (D / 16) + (d >> 4)) * 2 + ((d >> 3) & 1)) * 32 + (j & 31)) * 8 +
         (d & 7);
}
// elements of one (plane, sequence, KV head) slab
__device__ __forceinline__ int64_t kbar_slab(int n_max, int D) {
  return (int64_t)((n_max + 31) / 32) * 32 * D;
}
template <int D>
__global__ __launch_bounds__(256) void kap_pool_keys(const KapParams p) {
  constexpr int NT = 256;
  constexpr int KCH = D / 8;          // 16-byte chunks per key row
  constexpr int RG = NT / KCH;        // row groups
  __shared__ float red[RG][D];

  // consecutive workgroups take the KV heads of one logical key block (p.ppb
  // pages of kPage keys), whose slices lie side by side in each page
  const int j = blockIdx.x / p.hkv;
  const int g = blockIdx.x - j * p.hkv;
  const int b = blockIdx.y;
  const int q0 = p.cu_seqlens[b];
  const int L = p.cu_seqlens[b + 1] - q0;
  if (j * p.kv_block >= L) return;
  const int nvalid = min(p.kv_block, L - j * p.kv_block);
  const int32_t* pt = p.page_table + (int64_t)b * p.max_pages + (int64_t)j * p.ppb;
  const int tid = threadIdx.x;
  const int c = tid % KCH;
  const int rg = tid / KCH;
  const float inv = 1.f / (float)nvalid;
  const int64_t slab = kbar_slab(p.n_max, D);
  const int64_t plane = (int64_t)p.batch * p.hkv * slab;

  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int r = rg; r < nvalid; r += RG) {
    const int page = pt[r / kPage];
    const uint16_t* base = p.k_pool + ((int64_t)page * p.hkv + g) * (kPage * D) + c * 8;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(base + (r % kPage) * D);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc[2 * w] += bf16_lo(v[w]);
      acc[2 * w + 1] += bf16_hi(v[w]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rg][c * 8 + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < RG; ++k) sum += red[k][tid];
    uint16_t hi, lo;
    split_bf16(sum * inv, hi, lo);
    const int64_t at = ((int64_t)b * p.hkv + g) * slab + kbar_offset<D>(j, tid);
    p.kbar[at] = hi;
    p.kbar[plane + at] = lo;
  }
}

// ---------------------------------------------------------------------------
// Online (max, arg-max, sum of exp2) triples, merged across lanes and waves.
struct RowStat {
  float m;   // max score (log2 units)
  float z;   // sum of exp2(score - m)
  int a;     // lowest block index reaching m
};
__device__ __forceinline__ RowStat merge(RowStat x, RowStat y) {
  RowStat o;
  o.m = fmaxf(x.m, y.m);
  const float ex = x.m == kNegInf ? 0.f : __builtin_amdgcn_exp2f(x.m - o.m);
  const float ey = y.m == kNegInf ? 0.f : __builtin_amdgcn_exp2f(y.m - o.m);
  o.z = x.z * ex + y.z * ey;
  o.a = x.m > y.m ? x.a : (y.m > x.m ? y.a : min(x.a, y.a));
  return o;
}

// A logical key block spans one or two pages (kv_block 64 or 128).
constexpr int kMaxPagesPerBlock = 2;

// Inclusive prefix (sum, min or max) over the 64 lanes of a wavefront in six
// DPP steps, without LDS: row_shr 1, 2, 4, 8 inside each row of 16 lanes
// (lanes shifted in from outside the row contribute the identity), then
// row_bcast:15 adds row r's last lane into row r + 1 (rows 1 and 3) and
// row_bcast:31 lane 31 into rows 2 and 3.  Lane 63 holds the whole wave's.
enum ScanOp { kScanAdd, kScanMin, kScanMax };
template <ScanOp OP>
__device__ __forceinline__ uint32_t scan_apply(uint32_t a, uint32_t b) {
  return OP == kScanAdd ? a + b : OP == kScanMin ? (a < b ? a : b) : (a > b ? a : b);
}
template <ScanOp OP>
__device__ __forceinline__ uint32_t wave_scan(uint32_t x) {
  constexpr int id = OP == kScanMin ? -1 : 0;   // identity (as the DPP "old" value)
  x = scan_apply<OP>(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x111, 0xf, 0xf, false));
  x = scan_apply<OP>(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x112, 0xf, 0xf, false));
  x = scan_apply<OP>(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x114, 0xf, 0xf, false));
  x = scan_apply<OP>(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x118, 0xf, 0xf, false));
  x = scan_apply<OP>(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x142, 0xa, 0xf, false));
  x = scan_apply<OP>(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x143, 0xc, 0xf, false));
  return x;
}
template <ScanOp OP>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_scan<OP>(x), 63);
}

// The value of lane ^ S (S = 1 .. 32) in VALU cross-lane moves: quad_perm for
// 1 and 2; within a row of 16, row_ror:12 brings lane i + 4 and row_ror:4
// lane i - 4 (so lane ^ 4 is a choice on lane bit 2) and row_ror:8 lane i ^ 8;
// v_permlane16_swap and v_permlane32_swap return the values of the lanes with
// that bit clear and set, of which the partner's is the other one.
template <int S>
__device__ __forceinline__ uint32_t lane_xor(uint32_t x, int lane) {
  if constexpr (S == 1) return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xf, 0xf, false);
  if constexpr (S == 2) return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xf, 0xf, false);
  if constexpr (S == 4) {
    const uint32_t up = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x12C, 0xf, 0xf, false);
    const uint32_t dn = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x124, 0xf, 0xf, false);
    return (lane & 4) ? dn : up;
  }
  if constexpr (S == 8) return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x128, 0xf, 0xf, false);
  if constexpr (S == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return (lane & 16) ? r[0] : r[1];
  }
  if constexpr (S == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return (lane & 32) ? r[0] : r[1];
  }
  return x;
}

// One compare-exchange stage of a bitonic network over 256 keys held as four
// per lane (key e * 64 + lane in v[e]): blocks of SIZE, partner at STRIDE;
// the lower key of a pair keeps the smaller one in ascending blocks.
template <int SIZE, int STRIDE>
__device__ __forceinline__ void bitonic_stage(unsigned long long (&v)[4], int lane) {
  if constexpr (STRIDE >= 64) {
    constexpr int se = STRIDE / 64;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (e & se) continue;
      const bool asc = ((e * 64) & SIZE) == 0;
      const unsigned long long a = v[e], b = v[e | se];
      const bool sw = (a > b) == asc;
      v[e] = sw ? b : a;
      v[e | se] = sw ? a : b;
    }
  } else {
    const bool lower = (lane & STRIDE) == 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool asc = ((e * 64 + lane) & SIZE) == 0;
      const uint32_t plo = lane_xor<STRIDE>((uint32_t)v[e], lane);
      const uint32_t phi = lane_xor<STRIDE>((uint32_t)(v[e] >> 32), lane);
      const unsigned long long pv = ((unsigned long long)phi << 32) | plo;
      const bool keep_min = lower == asc;
      const bool take = keep_min ? pv < v[e] : pv > v[e];
      v[e] = take ? pv : v[e];
    }
  }
}

// Ascending sort of the first NPOW (power of two, 64 .. 256) of four keys per
// lane: the bitonic network's stages for block sizes up to NPOW.
template <int SIZE>
__device__ __forceinline__ void bitonic_sizes(unsigned long long (&v)[4], int lane, int npow) {
  if constexpr (SIZE <= 256) {
    if (SIZE > npow) return;
    if constexpr (SIZE >= 256) bitonic_stage<SIZE, 128>(v, lane);
    if constexpr (SIZE >= 128) bitonic_stage<SIZE, 64>(v, lane);
    if constexpr (SIZE >= 64) bitonic_stage<SIZE, 32>(v, lane);
    if constexpr (SIZE >= 32) bitonic_stage<SIZE, 16>(v, lane);
    if constexpr (SIZE >= 16) bitonic_stage<SIZE, 8>(v, lane);
    if constexpr (SIZE >= 8) bitonic_stage<SIZE, 4>(v, lane);
    if constexpr (SIZE >= 4) bitonic_stage<SIZE, 2>(v, lane);
    bitonic_stage<SIZE, 1>(v, lane);
    bitonic_sizes<SIZE * 2>(v, lane, npow);
  }
}

// Top-p mass of a key in fixed point: the key's w rounded down to a multiple
// of 2^-48 (w * 2^48 is exact in fp32, the conversion truncates).
__device__ __forceinline__ unsigned long long key_mass(uint32_t key_hi) {
  const float w = __uint_as_float(0x7FFFFFFFu - (key_hi & 0x7FFFFFFFu));
  return (unsigned long long)(w * 281474976710656.0f);
}

// HPW = 1: one query head, kTilesPerGroup consecutive tiles per workgroup,
// one mask row per (sequence, query head, tile).  HPW > 1: the HPW query
// heads of one KV head, one tile per workgroup, one mask row per (sequence,
// KV head, tile) shared by those heads (their proxy rows scored together).
template <int D, int R, bool kTopP, int HPW>
__global__ __launch_bounds__(256, 2) void kap_select(const KapParams p) {
  constexpr int NT = 256;
  constexpr int NWAVE = NT / 64;
  constexpr bool kShared = HPW > 1;
  constexpr int TPW = kShared ? 1 : kTilesPerGroup;
  constexpr int RPT = HPW * R;                // proxy rows per tile
  constexpr int MR = TPW * RPT;               // proxy rows of the workgroup (<= 32)
  constexpr int BQ = R * kProxyRows;
  constexpr int KSTEPS = D / 16;
  constexpr int KCH = D / 8;
  static_assert(MR <= 32, "one 32-row MFMA operand");

  // 16 KB of sort keys per tile.  Before the keys are built the same space
  // holds the pooled queries (2 x 32 rows of D bf16, each row padded by 16
  // bytes so that the 32 rows' operand reads of one k-step fall on different
  // banks), then the partial row statistics of pass 1 (max, sum, arg-max:
  // 32 rows x kParts each).
  constexpr int kParts = 2 * NWAVE;           // partials per row: lane halves x waves
  constexpr int kQRow = D + 8;
  // A tile's keys start one 8-byte key further along the banks than the
  // tile before's: a pass-2 key write of a wavefront puts 16 keys of each
  // tile at even (or odd) key positions modulo 32, the same for every tile,
  // which the odd offset spreads over both halves of the banks.
  constexpr int kKeyStride = kMaxCandidates + 1;
  constexpr int kKeyWords = TPW * kKeyStride;
  constexpr int kPartWords = (3 * 32 * kParts + 1) / 2;
  constexpr int kQWords = 2 * 32 * kQRow * 2 / 8;
  constexpr int kRawWords = kKeyWords > kPartWords ? (kKeyWords > kQWords ? kKeyWords : kQWords)
                                                   : (kPartWords > kQWords ? kPartWords : kQWords);
  __shared__ __attribute__((aligned(16))) unsigned long long sKeyRaw[kRawWords];
  auto sKey = reinterpret_cast<unsigned long long (*)[kKeyStride]>(sKeyRaw);
  __shared__ float sRowM[32];
  __shared__ float sRowInvZ[32];
  __shared__ int sHrm[TPW];          // HRM keys per tile
  __shared__ int sTopK[TPW];         // Top-p: kept count per tile
  __shared__ __attribute__((aligned(16))) uint32_t sHist[NWAVE][256];
  __shared__ unsigned long long sMass[kTopP ? NWAVE : 1][256];   // Top-p only
  static_assert(2 * 32 * kQRow * 2 <= (int)sizeof(sKeyRaw), "pooled queries fit");
  uint16_t* sQhi = reinterpret_cast<uint16_t*>(sKeyRaw);
  uint16_t* sQlo = sQhi + 32 * kQRow;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hf = lane >> 5;
  const int col = lane & 31;

  // One (sequence, KV head) after the other, so that the concurrently running
  // workgroups share that head's pooled keys (1 MB at 128K) in L2; inside it
  // the tile groups with the most candidates first, the query heads of the
  // GQA group side by side.
  const int ngroups = (p.nqb + TPW - 1) / TPW;
  const int hg = p.hq / p.hkv;
  const int per_kv = kShared ? ngroups : ngroups * hg;
  const int local = blockIdx.x / per_kv;
  const int G = p.group_begin + local;
  const int rem = blockIdx.x - local * per_kv;
  const int level = kShared ? rem : rem / hg;
  const int b = G / p.hkv;
  const int g = G - b * p.hkv;
  const int h = kShared ? g * hg : g * hg + (rem - level * hg);   // first (or only) head
  const int i0 = (ngroups - 1 - level) * TPW;
  // mask rows: (b, query head) or (b, KV head)
  const int64_t mrow0 = kShared ? ((int64_t)b * p.hkv + g) * p.nqb
                                : ((int64_t)b * p.hq + h) * p.nqb;
  const int q0 = p.cu_seqlens[b];
  const int L = p.cu_seqlens[b + 1] - q0;
  const int kvb = p.kv_block;
  const int32_t* __restrict__ pt = p.page_table + (int64_t)b * p.max_pages;

  // per-tile sizes (n = 0 for a tile past the sequence's end)
  int n_t[TPW], rows_t[TPW];
  int n_wg = 0;
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int i = i0 + t;
    const bool valid = i < p.nqb && i * BQ < L;
    n_t[t] = valid ? (min((i + 1) * BQ, L) - 1) / kvb + 1 : 0;
    rows_t[t] = valid ? HPW * min(R, (L - i * BQ + kProxyRows - 1) / kProxyRows) : 0;
    n_wg = max(n_wg, n_t[t]);
  }
  // rows that are past the end of the sequence (or of the group) have no
  // candidates; cand(m) = number of candidate blocks of proxy row m
  // proxy row m: tile m / RPT, head (m / R) % HPW, row m % R of that tile
  auto row_cand = [&](int m) -> int {
    if (m >= MR) return 0;
    const int i = i0 + m / RPT;
    const int start = i * BQ + (m % R) * kProxyRows;
    if (i >= p.nqb || start >= L) return 0;
    return (min(start + kProxyRows, L) - 1) / kvb + 1;
  };

  if (n_wg == 0) {
    for (int t = 0; t < TPW; ++t) {
      const int i = i0 + t;
      if (i >= p.nqb) break;
      const int64_t row = mrow0 + i;
      for (int s = tid; s < p.capacity; s += NT) p.ordered_blocks[row * p.capacity + s] = -1;
      for (int s = tid; s < p.capacity * p.ppb; s += NT)
        p.ordered_pages[row * p.capacity * p.ppb + s] = -1;
      if (tid == 0) {
        p.counts[row] = 0;
        if (p.hrm_counts != nullptr) p.hrm_counts[row] = 0;
      }
      if (p.debug_w != nullptr)
        for (int jj = tid; jj < p.n_max; jj += NT) p.debug_w[row * p.n_max + jj] = 0.f;
      if (p.debug_hrm != nullptr)
        for (int jj = tid; jj < p.n_max; jj += NT) p.debug_hrm[row * p.n_max + jj] = 0;
    }
    return;
  }

  // ---- 1) pooled queries (mean of 16 rows, times scale*log2e), split bf16.
  // Every load of a thread is issued before the first add (no dependent
  // HBM round trips).
  {
    constexpr int PAIRS = 32 * KCH / NT;           // (row, 16-byte chunk) pairs per thread
    static_assert(32 * KCH % NT == 0, "pairs split evenly");
    const float qscale = p.scale * kLog2e;
    u32x4_t v[PAIRS][kProxyRows];
    int nrow[PAIRS];
#pragma unroll
    for (int e = 0; e < PAIRS; ++e) {
      const int idx = tid + e * NT;
      const int m = idx / KCH, c = idx % KCH;
      nrow[e] = 0;
      int start = 0;
      if (m < MR && i0 + m / RPT < p.nqb) {
        start = (i0 + m / RPT) * BQ + (m % R) * kProxyRows;
        nrow[e] = max(min(start + kProxyRows, L) - start, 0);
      }
      const int hq_m = h + (m / R) % HPW;   // the row's query head
      const uint16_t* src = p.q + ((int64_t)(q0 + start) * p.hq + hq_m) * D + c * 8;
#pragma unroll
      for (int t = 0; t < kProxyRows; ++t) {
        v[e][t] = (u32x4_t){0u, 0u, 0u, 0u};
        if (t < nrow[e]) v[e][t] = *reinterpret_cast<const u32x4_t*>(src + (int64_t)t * p.hq * D);
      }
    }
#pragma unroll
    for (int e = 0; e < PAIRS; ++e) {
      const int idx = tid + e * NT;
      const int m = idx / KCH, c = idx % KCH;
      float acc[8];
#pragma unroll
      for (int x = 0; x < 8; ++x) acc[x] = 0.f;
#pragma unroll
      for (int t = 0; t < kProxyRows; ++t)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          acc[2 * w] += bf16_lo(v[e][t][w]);
          acc[2 * w + 1] += bf16_hi(v[e][t][w]);
        }
      const float f = nrow[e] > 0 ? qscale / (float)nrow[e] : 0.f;
      u32x4_t hv, lv;   // the 8 values of the chunk, one 16-byte store per plane
#pragma unroll
      for (int x = 0; x < 8; x += 2) {
        uint16_t h0, l0, h1, l1;
        split_bf16(acc[x] * f, h0, l0);
        split_bf16(acc[x + 1] * f, h1, l1);
        hv[x / 2] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        lv[x / 2] = (uint32_t)l0 | ((uint32_t)l1 << 16);
      }
      *reinterpret_cast<u32x4_t*>(&sQhi[m * kQRow + c * 8]) = hv;
      *reinterpret_cast<u32x4_t*>(&sQlo[m * kQRow + c * 8]) = lv;
    }
  }
  __syncthreads();

  // ---- 2) A operand (pooled queries, rows x d) into registers
  bf16x8_t ahi[KSTEPS], alo[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    ahi[ks] = *reinterpret_cast<const bf16x8_t*>(&sQhi[col * kQRow + ks * 16 + hf * 8]);
    alo[ks] = *reinterpret_cast<const bf16x8_t*>(&sQlo[col * kQRow + ks * 16 + hf * 8]);
  }
  // every wave holds its operand before any wave writes the partial row
  // statistics into the same LDS space (a wave without candidate blocks
  // writes them right away)
  __syncthreads();

  const int64_t slab = kbar_slab(p.n_max, D);
  const int64_t plane = (int64_t)p.batch * p.hkv * slab;
  const uint16_t* kb_hi = p.kbar + ((int64_t)b * p.hkv + g) * slab;
  const uint16_t* kb_lo = kb_hi + plane;
  const int nb = (n_wg + 31) / 32;

  // pooled-key operands of candidate block group cb; a wave loads a group
  // while the products of the group before it run and the statistics of the
  // one before that are updated
  bf16x8_t kh[KSTEPS], kl[KSTEPS];
  // (blocks past the sequence's last one hold stale values; their scores
  // are masked)
  auto load_ops = [&](int cb) {
    const int64_t at = kbar_offset<D>(cb * 32 + col, hf * 8);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      kh[ks] = *reinterpret_cast<const bf16x8_t*>(kb_hi + at + ks * (2 * 32 * 8));
      kl[ks] = *reinterpret_cast<const bf16x8_t*>(kb_lo + at + ks * (2 * 32 * 8));
    }
  };
  // Scores of the loaded group for the 32 proxy rows (log2 units). With the
  // blocks as the rows of the result (block_rows), lane (col, hf) holds
  // proxy row col for the blocks 8(r/4) + 4hf + r%4 of the group; otherwise
  // block col for the proxy rows 8(r/4) + 4hf + r%4. With load_next, each
  // k-step's operands are replaced by those of group `next` as soon as its
  // three products have read them (the loads then have the rest of the
  // chain as lead time; the interleave is pinned, since the scheduler would
  // otherwise move every load behind the last product).
  auto scores = [&](auto block_rows, auto load_next, int next) -> f32x16_t {
    constexpr bool kBlockRows = decltype(block_rows)::value;
    constexpr bool kLoadNext = decltype(load_next)::value;
    f32x16_t acc = {};
    const int64_t at = kbar_offset<D>(next * 32 + col, hf * 8);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      if constexpr (kBlockRows) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kh[ks], ahi[ks], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kl[ks], ahi[ks], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kh[ks], alo[ks], acc, 0, 0, 0);
      } else {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi[ks], kh[ks], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi[ks], kl[ks], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo[ks], kh[ks], acc, 0, 0, 0);
      }
      if constexpr (kLoadNext) {
        kh[ks] = *reinterpret_cast<const bf16x8_t*>(kb_hi + at + ks * (2 * 32 * 8));
        kl[ks] = *reinterpret_cast<const bf16x8_t*>(kb_lo + at + ks * (2 * 32 * 8));
        __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);   // three MFMAs
        __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);   // then two vector loads
      }
    }
    return acc;
  };
  constexpr std::true_type kRowsAreBlocks{}, kLoadNextGroup{};
  constexpr std::false_type kRowsAreProxyRows{}, kNoLoad{};
  // "have rowmax" flags as a bitmap per tile (in the radix histogram space,
  // which is free until the selection)
  // ([kMaxCandidates / 32][TPW]: one group's words of every tile side by side)
  uint32_t* sHrmBits = &sHist[0][0];
  static_assert(TPW * (kMaxCandidates / 32) <= NWAVE * 256, "bitmap fits");
  for (int x = tid; x < TPW * (kMaxCandidates / 32); x += NT) sHrmBits[x] = 0u;
  if (tid < TPW) sHrm[tid] = 0;   // HRM keys per tile, counted as the flags are set

  // ---- 3) pass 1: per-row max, arg-max (lowest block) and sum, online.
  // The products put the blocks on the rows, so lane (col, hf) keeps the
  // statistics of proxy row col over its half of every group: blocks
  // 8(r/4) + 4hf + r%4 for r = 0..15, in ascending order.
  const int cand_raw = row_cand(col);
  const bool row_ok = cand_raw > 0;
  // a row without candidates runs the unmasked path on whatever it reads;
  // its statistics are dropped before the merge
  const int cand_l = row_ok ? cand_raw : 0x3FFFFFFF;
  RowStat st{kNegInf, 0.f, 0x7FFFFFFF};
  // software-pipelined: the products of group cb + NWAVE are issued before
  // the statistics of group cb, whose vector work then overlaps them, and
  // the operands of group cb + 2 NWAVE are loaded meanwhile (near the end
  // the index is clamped to the last group; that load goes unused)
  auto stats1 = [&](const f32x16_t& acc, int cb) {
    // element r is block cb * 32 + 4hf + off(r), off(r) = 8(r/4) + r%4 <= 27
    const int lim = cand_l - cb * 32 - 4 * hf;
    float sv[16];
    if (__all(lim >= 28)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sv[r] = acc[r];
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) sv[r] = 8 * (r >> 2) + (r & 3) < lim ? acc[r] : kNegInf;
    }
    float mx = fmaxf(sv[0], sv[1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) mx = fmaxf(fmaxf(mx, sv[r]), sv[r + 1]);
    const float mn = fmaxf(st.m, mx);
    const float mu = mn == kNegInf ? 0.f : mn;   // no valid score yet: every term is 0
    float e[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) e[r] = __builtin_amdgcn_exp2f(sv[r] - mu);
#pragma unroll
    for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
      for (int r = 0; r < w; ++r) e[r] += e[r + w];
    const float zn = fmaf(st.z, __builtin_amdgcn_exp2f(st.m - mu), e[0]);
    if (__any(mx > st.m)) {
      // a strict raise takes the group's lowest block reaching the new max
      // (an equal max keeps the earlier, lower block)
      int ai = 0x7FFFFFFF;
#pragma unroll
      for (int r = 15; r >= 0; --r)
        ai = sv[r] == mx ? cb * 32 + 4 * hf + 8 * (r >> 2) + (r & 3) : ai;
      st.a = mx > st.m ? ai : st.a;
    }
    st.m = mn;
    st.z = zn;
  };
  f32x16_t acc_cur = {};
  if (wave < nb) {
    load_ops(wave);
    acc_cur = scores(kRowsAreBlocks, kNoLoad, 0);
    if (wave + NWAVE < nb) load_ops(wave + NWAVE);
  }
  int cb1 = wave;
  for (; cb1 + NWAVE < nb; cb1 += NWAVE) {
    const f32x16_t acc_next = scores(kRowsAreBlocks, kLoadNextGroup, min(cb1 + 2 * NWAVE, nb - 1));
    stats1(acc_cur, cb1);
    acc_cur = acc_next;
  }
  if (cb1 < nb) stats1(acc_cur, cb1);
  // merge the kParts partial statistics of every row (two lane halves x
  // NWAVE waves): eight threads per row, one partial each (max first, then
  // the sum rescaled to it and the lowest block index reaching it), combined
  // over three lane steps
  static_assert(kParts == 8, "one partial per thread of a row");
  float* sPm = reinterpret_cast<float*>(sKeyRaw);
  float* sPz = sPm + 32 * kParts;
  int* sPa = reinterpret_cast<int*>(sPz + 32 * kParts);
  {
    const int at = col * kParts + wave * 2 + hf;
    sPm[at] = row_ok ? st.m : kNegInf;
    sPz[at] = row_ok ? st.z : 0.f;
    sPa[at] = row_ok ? st.a : 0x7FFFFFFF;
  }
  __syncthreads();
  {
    const int row = tid >> 3;
    const int at = row * kParts + (tid & 7);
    RowStat s{sPm[at], sPz[at], sPa[at]};
    // combine the eight threads of the row: with lane ^ 1 and lane ^ 2
    // (quad_perm), then each quad with the other quad of its eight lanes
    // (row_half_mirror pairs lane i with 7 - i) -- the tree of an xor
    // butterfly, in DPP moves
#pragma unroll
    for (int lvl = 0; lvl < 3; ++lvl) {
      auto partner = [&](int v) -> int {
        return lvl == 0 ? __builtin_amdgcn_mov_dpp(v, 0xB1, 0xf, 0xf, false)
               : lvl == 1 ? __builtin_amdgcn_mov_dpp(v, 0x4E, 0xf, 0xf, false)
                          : __builtin_amdgcn_mov_dpp(v, 0x141, 0xf, 0xf, false);
      };
      RowStat o;
      o.m = __int_as_float(partner(__float_as_int(s.m)));
      o.z = __int_as_float(partner(__float_as_int(s.z)));
      o.a = partner(s.a);
      s = merge(s, o);
    }
    if ((tid & 7) == 0) {
      sRowM[row] = s.m;
      sRowInvZ[row] = s.z > 0.f ? 1.f / s.z : 0.f;
      if (s.m != kNegInf && row < MR) {
        const int t = row / RPT;
        const uint32_t bit = 1u << (s.a & 31);
        if ((atomicOr(&sHrmBits[(s.a >> 5) * TPW + t], bit) & bit) == 0u) atomicAdd(&sHrm[t], 1);
      }
    }
  }
  __syncthreads();

  // ---- 4) pass 2: importance w and HRM flag per (tile, candidate) -> keys
  // w = the sum over the tile's proxy rows / their count, as a product with
  // the reciprocal (exact for the usual power-of-two count)
  float inv_rows[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) inv_rows[t] = rows_t[t] > 0 ? 1.f / (float)rows_t[t] : 0.f;
  // key of block j of tile t (~0 past the tile's candidates); hrm: block j
  // is flagged for tile t
  auto emit = [&](int t, int j, int n, float inv, float wsum, bool hrm) {
    unsigned long long key = ~0ull;
    if (j < n) {
      const float w = wsum * inv;
      const uint32_t wb = __float_as_uint(w);   // w >= 0: bit order == value order
      key = ((unsigned long long)(hrm ? 0u : 1u) << 63) |
            ((unsigned long long)(0x7FFFFFFFu - wb) << 32) | (uint32_t)j;
      const int64_t row = mrow0 + i0 + t;
      if (p.debug_w != nullptr) p.debug_w[row * p.n_max + j] = w;
      if (p.debug_hrm != nullptr) p.debug_hrm[row * p.n_max + j] = hrm ? 1 : 0;
    }
    sKey[t][j] = key;   // j < nb * 32 <= kMaxCandidates
  };
  // software-pipelined like pass 1
  if constexpr (!kShared) {
    // The products put the blocks on the rows as in pass 1: lane (col, hf)
    // holds proxy row col (tile col / R) for blocks 8(r/4) + 4hf + r%4 of
    // the group. A tile's weight of a block is the sum over its R lanes
    // (same hf), taken as a reduce-scatter: at each lane step the two
    // partners keep complementary halves of the remaining blocks, so that
    // each lane ends with 16 / R finished sums.
    const bool lane_row = col < MR;
    const int t_l = lane_row ? col / R : 0;
    int n_l = 0;
    float inv_l = 0.f;
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      n_l = t_l == t ? n_t[t] : n_l;
      inv_l = t_l == t ? inv_rows[t] : inv_l;
    }
    const float rm_l = sRowM[col];
    const float riz_l = sRowInvZ[col];
    const int cand_l2 = lane_row ? row_cand(col) : 0;
    __syncthreads();
    constexpr int EPL = 16 / R;   // finished sums per lane
    auto weights_t = [&](const f32x16_t& acc, int cb, uint32_t hword) {
      // element r is block cb * 32 + 4hf + off(r), off(r) = 8(r/4) + r%4 <= 27
      const int lim = cand_l2 - cb * 32 - 4 * hf;
      float v[16];
      if (__all(lim >= 28)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] = __builtin_amdgcn_exp2f(acc[r] - rm_l) * riz_l;
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          v[r] = 8 * (r >> 2) + (r & 3) < lim ? __builtin_amdgcn_exp2f(acc[r] - rm_l) * riz_l : 0.f;
      }
      // lane steps: lane bit 2 against the mirror lane 7 - i (R == 8 only),
      // then bit 1 (lane ^ 2), then bit 0 (lane ^ 1); the lane with the bit
      // set keeps the upper half
      int base = 0;
      auto step = [&](auto n_c, auto ctrl_c, int bit) {
        constexpr int N = decltype(n_c)::value;
        constexpr int CTRL = decltype(ctrl_c)::value;
        const bool up = (col >> bit) & 1;
#pragma unroll
        for (int x = 0; x < N / 2; ++x) {
          const float send = up ? v[x] : v[x + N / 2];
          const float keep = up ? v[x + N / 2] : v[x];
          v[x] = keep + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(send), CTRL, 0xf, 0xf, false));
        }
        base += up ? N / 2 : 0;
      };
      if constexpr (R == 8) {
        step(std::integral_constant<int, 16>{}, std::integral_constant<int, 0x141>{}, 2);
        step(std::integral_constant<int, 8>{}, std::integral_constant<int, 0x4E>{}, 1);
        step(std::integral_constant<int, 4>{}, std::integral_constant<int, 0xB1>{}, 0);
      } else {
        static_assert(R == 4, "four or eight proxy rows per tile");
        step(std::integral_constant<int, 16>{}, std::integral_constant<int, 0x4E>{}, 1);
        step(std::integral_constant<int, 8>{}, std::integral_constant<int, 0xB1>{}, 0);
      }
      if (lane_row) {
#pragma unroll
        for (int x = 0; x < EPL; ++x) {
          const int r = base + x;
          const int j = cb * 32 + 4 * hf + 8 * (r >> 2) + (r & 3);
          emit(t_l, j, n_l, inv_l, v[x], (hword >> (j & 31)) & 1u);
        }
      }
    };
    acc_cur = (f32x16_t){};
    if (wave < nb) {
      load_ops(wave);
      acc_cur = scores(kRowsAreBlocks, kNoLoad, 0);
      if (wave + NWAVE < nb) load_ops(wave + NWAVE);
    }
    int cb2 = wave;
    for (; cb2 + NWAVE < nb; cb2 += NWAVE) {
      // the group's HRM bitmap word of the lane's tile, read ahead of the
      // products
      const uint32_t hword = sHrmBits[cb2 * TPW + t_l];
      __builtin_amdgcn_sched_barrier(0);
      const f32x16_t acc_next =
          scores(kRowsAreBlocks, kLoadNextGroup, min(cb2 + 2 * NWAVE, nb - 1));
      weights_t(acc_cur, cb2, hword);
      acc_cur = acc_next;
    }
    if (cb2 < nb) weights_t(acc_cur, cb2, sHrmBits[cb2 * TPW + t_l]);
  } else {
    // One tile of HPW query heads: the products put the proxy rows on the
    // rows, lane (col, hf) holds block col of the group for rows
    // m = 8(r/4) + 4hf + r%4, and the tile's weight is a sum inside the lane
    // plus one lane swap.
    int cand[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) cand[r] = row_cand(8 * (r >> 2) + 4 * hf + (r & 3));
    float rm[16], riz[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 8 * (r >> 2) + 4 * hf + (r & 3);
      rm[r] = sRowM[m];
      riz[r] = sRowInvZ[m];
    }
    __syncthreads();
    auto weights = [&](const f32x16_t& acc, int cb, uint32_t hword) {
      const int j = cb * 32 + col;
      const bool hrm = (hword >> col) & 1u;
      float part[4];
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        float sum = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g4 + e;
          sum += j < cand[r] ? __builtin_amdgcn_exp2f(acc[r] - rm[r]) * riz[r] : 0.f;
        }
        part[g4] = sum;
      }
      const float wt = pair_sum(part[0] + part[1] + part[2] + part[3]);
      if (hf == 0) emit(0, j, n_t[0], inv_rows[0], wt, hrm);
    };
    acc_cur = (f32x16_t){};
    if (wave < nb) {
      load_ops(wave);
      acc_cur = scores(kRowsAreProxyRows, kNoLoad, 0);
      if (wave + NWAVE < nb) load_ops(wave + NWAVE);
    }
    int cb2 = wave;
    for (; cb2 + NWAVE < nb; cb2 += NWAVE) {
      const uint32_t hword = sHrmBits[cb2];
      __builtin_amdgcn_sched_barrier(0);
      const f32x16_t acc_next =
          scores(kRowsAreProxyRows, kLoadNextGroup, min(cb2 + 2 * NWAVE, nb - 1));
      weights(acc_cur, cb2, hword);
      acc_cur = acc_next;
    }
    if (cb2 < nb) weights(acc_cur, cb2, sHrmBits[cb2]);
  }
  __syncthreads();

  // ---- 5) top-k selection per tile (wave t handles tile t): radix-select
  // the k-th smallest key on its upper 32 bits (HRM flag and -w), keep every
  // key below that value and every key equal to it (ties are broken by the
  // block index in the sort that follows), compacted in place.
  static_assert(TPW <= NWAVE, "one wave per tile of the group");
  int k_t[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int n = n_t[t];
    int k = 0;
    if (n > 0) {
      const long long kk = ((long long)n * p.beta_ppm + 999999) / 1000000;
      k = (int)(kk < 1 ? 1 : (kk > n ? n : kk));
    }
    k_t[t] = k;
  }
  if (wave < TPW) {
    const int t = wave;
    const int n = n_t[t];
    int k = k_t[t];
    int sel = n;                              // keys kept for the final sort
    // upper key halves (HRM flag, -w) of the tile, lane + 64e, in registers
    // for the radix rounds
    constexpr int kPerLane = kMaxCandidates / 64;
    uint32_t hk[kPerLane];
    const uint32_t* khalf = reinterpret_cast<const uint32_t*>(&sKey[t][0]);
#pragma unroll
    for (int e = 0; e < kPerLane; ++e) {
      const int idx = lane + 64 * e;
      hk[e] = idx < n ? khalf[2 * idx + 1] : 0u;
    }
    uint32_t top_prefix = 0;
    bool top_bound = false;                   // the Top-p count decides k
    if (kTopP && n > 0 && k > 1) {
      // Top-p: the smallest k whose leading keys (ascending key order = the
      // visiting order) carry at least the fixed-point mass P.  Radix descent
      // over the upper 32 key bits with per-digit counts and exact integer
      // masses; the last digit leaves a group of keys with equal w (same
      // upper bits) ordered by block index, of which just enough are taken.
      unsigned long long need = p.top_p_fx;
      uint32_t prefix = 0, pmask = 0;
      int before_cnt = 0;
      bool reached = true;
      for (int shift = 24; shift >= 0 && reached; shift -= 8) {
        for (int bin = lane; bin < 256; bin += 64) {
          sHist[t][bin] = 0;
          sMass[t][bin] = 0ull;
        }
#pragma unroll
        for (int e = 0; e < kPerLane; ++e) {
          if (64 * e >= n) break;
          const uint32_t hi = hk[e];
          if (lane + 64 * e < n && (hi & pmask) == prefix) {
            const uint32_t d = (hi >> shift) & 255u;
            atomicAdd(&sHist[t][d], 1u);
            atomicAdd(&sMass[t][d], key_mass(hi));
          }
        }
        uint32_t c[4];
        unsigned long long m[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          c[e] = sHist[t][4 * lane + e];
          m[e] = sMass[t][4 * lane + e];
        }
        const uint32_t cmine = c[0] + c[1] + c[2] + c[3];
        const unsigned long long mmine = m[0] + m[1] + m[2] + m[3];
        uint32_t cincl = cmine;
        unsigned long long mincl = mmine;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const uint32_t oc = __shfl_up(cincl, off);
          const unsigned long long om = __shfl_up(mincl, off);
          if (lane >= off) {
            cincl += oc;
            mincl += om;
          }
        }
        uint32_t cbefore = cincl - cmine;
        unsigned long long mbefore = mincl - mmine;
        int digit = -1, cnt_left = 0;
        unsigned long long need_left = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (digit < 0 && mbefore < need && mbefore + m[e] >= need) {
            digit = 4 * lane + e;
            cnt_left = (int)cbefore;
            need_left = need - mbefore;
          }
          cbefore += c[e];
          mbefore += m[e];
        }
        const unsigned long long found = __ballot(digit >= 0);
        if (found == 0ull) {
          reached = false;   // the whole tile holds less than P: every key
        } else {
          const int src = __ffsll((long long)found) - 1;
          digit = __shfl(digit, src);
          before_cnt += __shfl(cnt_left, src);
          need = __shfl(need_left, src);
          prefix |= (uint32_t)digit << shift;
          pmask |= 0xFFu << shift;
        }
      }
      if (reached) {
        const unsigned long long wq = key_mass(prefix);   // > 0: its group holds need > 0
        const int kp = before_cnt + (int)((need + wq - 1) / wq);
        if (kp < k) {
          k = kp;
          top_bound = true;
          top_prefix = prefix;
        }
      }
      if (lane == 0) sTopK[t] = k;
    }
    if (n > 0 && k < n) {
      uint32_t prefix = top_prefix, pmask = top_bound ? 0xFFFFFFFFu : 0u;
      int need = k;
      int nbits = 0;   // low bits of the k-th key still to resolve
      if (!top_bound) {
        // The upper halves begin with the HRM flag and the leading exponent
        // bits of -w, which most keys share, so a radix over fixed 8-bit
        // digits would send nearly every key of its first round to one or two
        // bins (same-address LDS atomics).  Instead, take the group (HRM or
        // not) that holds the k-th key, the lowest and highest key of that
        // group, and start the radix at the highest bit where they differ.
        const int h = sHrm[t];
        const uint32_t grp = k <= h ? 0u : 1u;
        uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
        for (int e = 0; e < kPerLane; ++e) {
          if (64 * e >= n) break;
          if (lane + 64 * e < n && (hk[e] >> 31) == grp) {
            lo = min(lo, hk[e]);
            hi = max(hi, hk[e]);
          }
        }
        lo = wave_reduce<kScanMin>(lo);
        hi = wave_reduce<kScanMax>(hi);
        const uint32_t diff = lo ^ hi;
        nbits = diff == 0u ? 0 : 32 - __clz((int)diff);
        pmask = nbits == 32 ? 0u : ~((1u << nbits) - 1u);
        prefix = lo & pmask;
        need = grp == 0u ? k : k - h;
      }
      while (nbits > 0) {
        const int width = nbits < 8 ? nbits : 8;
        const int shift = nbits - width;
        const uint32_t dmask = (1u << width) - 1u;
        for (int bin = lane; bin < 256; bin += 64) sHist[t][bin] = 0;
#pragma unroll
        for (int e = 0; e < kPerLane; ++e) {
          if (64 * e >= n) break;
          if (lane + 64 * e < n && (hk[e] & pmask) == prefix)
            atomicAdd(&sHist[t][(hk[e] >> shift) & dmask], 1u);
        }
        uint32_t c[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) c[e] = sHist[t][4 * lane + e];
        const uint32_t mine = c[0] + c[1] + c[2] + c[3];
        const uint32_t incl = wave_scan<kScanAdd>(mine);
        uint32_t before = incl - mine;
        int digit = -1, left = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (digit < 0 && before < (uint32_t)need && before + c[e] >= (uint32_t)need) {
            digit = 4 * lane + e;
            left = need - (int)before;
          }
          before += c[e];
        }
        const unsigned long long found = __ballot(digit >= 0);
        const int src = __ffsll((long long)found) - 1;   // uniform
        digit = __builtin_amdgcn_readlane(digit, src);
        need = __builtin_amdgcn_readlane(left, src);
        prefix |= (uint32_t)digit << shift;
        pmask |= dmask << shift;
        nbits = shift;
      }
      // compact keys with upper half <= prefix to the front, keeping order;
      // from the register copy (key idx is its upper half and idx itself)
      int written = 0;
#pragma unroll
      for (int e = 0; e < kPerLane; ++e) {
        if (64 * e >= n) break;
        const int idx = lane + 64 * e;
        const bool keep = idx < n && hk[e] <= prefix;
        const unsigned long long bal = __ballot(keep);
        const int pos = written + __popcll(bal & ((1ull << lane) - 1ull));
        if (keep) sKey[t][pos] = ((unsigned long long)hk[e] << 32) | (uint32_t)idx;
        written += __popcll(bal);
      }
      sel = written;
    }

    // ---- 6) bitonic sort of the kept keys, ascending, by this wavefront
    // alone: up to 256 keys in registers (four per lane, the cross-lane
    // partners by DPP and lane swaps), more in LDS (LDS operations of one
    // wavefront complete in order, so a step sees the writes of the step
    // before it without a workgroup barrier)
    int npow = 1;
    while (npow < sel) npow <<= 1;
    if (npow <= 256) {
      unsigned long long v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int idx = e * 64 + lane;
        v[e] = idx < sel ? sKey[t][idx] : ~0ull;
      }
      bitonic_sizes<2>(v, lane, npow);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int idx = e * 64 + lane;
        if (idx < npow) sKey[t][idx] = v[e];
      }
      npow = 0;   // nothing left for the LDS network
    }
    for (int j = sel + lane; j < npow; j += 64) sKey[t][j] = ~0ull;
    const int half = npow >> 1;
    for (int size = 2; size <= npow; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        for (int q = lane; q < half; q += 64) {
          const int lo = ((q & ~(stride - 1)) << 1) | (q & (stride - 1));
          const int hi = lo + stride;
          const bool up = (lo & size) == 0;
          const unsigned long long a = sKey[t][lo], c = sKey[t][hi];
          if ((a > c) == up) {
            sKey[t][lo] = c;
            sKey[t][hi] = a;
          }
        }
      }
    }
  }
  __syncthreads();
  if (kTopP) {
#pragma unroll
    for (int t = 0; t < TPW; ++t)
      if (n_t[t] > 0 && k_t[t] > 1) k_t[t] = sTopK[t];
  }

  // ---- 7) first k entries of every tile, remapped pages, counts.  The page
  // ids of one chunk of entries of every tile are loaded before any of the
  // chunk's stores: loads and stores share one counter, so a load issued after
  // a store would wait for that store.
  for (int s0 = 0; s0 < p.capacity; s0 += NT) {
    const int s = s0 + tid;
    int blk[TPW], pg[TPW][kMaxPagesPerBlock];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      blk[t] = -1;
      if (s < p.capacity && s < k_t[t]) blk[t] = (int)(sKey[t][s] & 0xFFFFFFFFu);
      // the block's pages; -1 for a page past the sequence's end
#pragma unroll
      for (int e = 0; e < kMaxPagesPerBlock; ++e) {
        pg[t][e] = -1;
        if (e < p.ppb && blk[t] >= 0 && blk[t] * kvb + e * kPage < L) pg[t][e] = pt[blk[t] * p.ppb + e];
      }
    }
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      if (i0 + t >= p.nqb || s >= p.capacity) continue;
      const int64_t row = mrow0 + i0 + t;
      p.ordered_blocks[row * p.capacity + s] = blk[t];
#pragma unroll
      for (int e = 0; e < kMaxPagesPerBlock; ++e)
        if (e < p.ppb) p.ordered_pages[(row * p.capacity + s) * p.ppb + e] = pg[t][e];
    }
  }
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int i = i0 + t;
    if (i >= p.nqb) break;
    const int64_t row = mrow0 + i;
    const int n = n_t[t];
    const int k = k_t[t];
    if (tid == 0) {
      p.counts[row] = k;
      if (p.hrm_counts != nullptr) p.hrm_counts[row] = min(k, sHrm[t]);
    }
    if (p.debug_w != nullptr)
      for (int jj = n + tid; jj < p.n_max; jj += NT) p.debug_w[row * p.n_max + jj] = 0.f;
    if (p.debug_hrm != nullptr)
      for (int jj = n + tid; jj < p.n_max; jj += NT) p.debug_hrm[row * p.n_max + jj] = 0;
  }
}

template <int D, int R>
hipError_t launch_kap_t(const KapParams& p, hipStream_t stream, KapStage stage) {
  const bool top_p = p.top_p_fx != 0;
  const int nkb = p.n_max;
  if (p.batch <= 0 || nkb <= 0) return hipSuccess;
  if (stage & kKapPool) {
    hipLaunchKernelGGL((kap_pool_keys<D>), dim3((unsigned)(nkb * p.hkv), p.batch), dim3(256), 0,
                       stream, p);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (!(stage & kKapSelect)) return hipSuccess;
  // workgroups per (sequence, KV head) group, times the groups launched
  const int64_t n_groups = p.group_count > 0 ? p.group_count : (int64_t)p.batch * p.hkv;
  if (p.shared_heads > 1) {
    const int64_t grid = n_groups * p.nqb;
#define COSA_KAP_SHARED(HPW_)                                                                \
  if constexpr (HPW_ * R <= 32) {                                                          \
    if (p.shared_heads == HPW_) {                                                          \
      if (top_p)                                                                           \
        hipLaunchKernelGGL((kap_select<D, R, true, HPW_>), dim3((unsigned)grid), dim3(256),  \
                           0, stream, p);                                                  \
      else                                                                                 \
        hipLaunchKernelGGL((kap_select<D, R, false, HPW_>), dim3((unsigned)grid), dim3(256), \
                           0, stream, p);                                                  \
      return hipGetLastError();                                                            \
    }                                                                                      \
  }
    COSA_KAP_SHARED(2)
    COSA_KAP_SHARED(4)
    COSA_KAP_SHARED(8)
#undef COSA_KAP_SHARED
    return hipErrorInvalidValue;
  }
  const int64_t groups = (p.nqb + kTilesPerGroup - 1) / kTilesPerGroup;
  const int64_t grid = n_groups * (p.hq / p.hkv) * groups;
  if (top_p)
    hipLaunchKernelGGL((kap_select<D, R, true, 1>), dim3((unsigned)grid), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((kap_select<D, R, false, 1>), dim3((unsigned)grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kap(const KapParams& p, int head_dim, int q_block, hipStream_t stream,
                      KapStage stage) {
  if (head_dim == 128 && q_block == 128) return launch_kap_t<128, 8>(p, stream, stage);
  if (head_dim == 128 && q_block == 64) return launch_kap_t<128, 4>(p, stream, stage);
  if (head_dim == 64 && q_block == 128) return launch_kap_t<64, 8>(p, stream, stage);
  if (head_dim == 64 && q_block == 64) return launch_kap_t<64, 4>(p, stream, stage);
  return hipErrorInvalidValue;
}

}  // namespace cosa
