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
//   kap_pool_keys  one workgroup per (sequence, key block): streams the page
//                  of every KV head once from HBM and writes the fp32 mean key
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

  const int j = blockIdx.x;   // logical key block (p.ppb pages of kPage keys)
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

  for (int g = 0; g < p.hkv; ++g) {
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
    __syncthreads();
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
  // holds the pooled queries (2 x 32 x D bf16), then the per-lane partial row
  // statistics of pass 1 (max, sum, arg-max: 32 rows x kPartStride each; the
  // stride spreads a row's partials over the LDS banks).
  constexpr int kPartStride = 32 * NWAVE + 8;
  constexpr int kKeyWords = TPW * kMaxCandidates;
  constexpr int kPartWords = (3 * 32 * kPartStride + 1) / 2;
  __shared__ __attribute__((aligned(16)))
  unsigned long long sKeyRaw[kKeyWords > kPartWords ? kKeyWords : kPartWords];
  auto sKey = reinterpret_cast<unsigned long long (*)[kMaxCandidates]>(sKeyRaw);
  __shared__ float sRowM[32];
  __shared__ float sRowInvZ[32];
  __shared__ int sHrm[TPW];          // HRM keys per tile
  __shared__ int sTopK[TPW];         // Top-p: kept count per tile
  __shared__ uint32_t sHist[NWAVE][256];
  __shared__ unsigned long long sMass[kTopP ? NWAVE : 1][256];   // Top-p only
  uint16_t* sQhi = reinterpret_cast<uint16_t*>(sKeyRaw);
  uint16_t* sQlo = sQhi + 32 * D;

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
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        uint16_t hi, lo;
        split_bf16(acc[x] * f, hi, lo);
        sQhi[m * D + c * 8 + x] = hi;
        sQlo[m * D + c * 8 + x] = lo;
      }
    }
  }
  __syncthreads();

  // ---- 2) A operand (pooled queries, rows x d) into registers
  bf16x8_t ahi[KSTEPS], alo[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    ahi[ks] = *reinterpret_cast<const bf16x8_t*>(&sQhi[col * D + ks * 16 + hf * 8]);
    alo[ks] = *reinterpret_cast<const bf16x8_t*>(&sQlo[col * D + ks * 16 + hf * 8]);
  }
  // every wave holds its operand before any wave writes the partial row
  // statistics into the same LDS space (a wave without candidate blocks
  // writes them right away)
  __syncthreads();
  // rows held by this lane's accumulator registers: m = 8(r/4) + 4hf + r%4
  int cand[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) cand[r] = row_cand(8 * (r >> 2) + 4 * hf + (r & 3));

  const int64_t slab = kbar_slab(p.n_max, D);
  const int64_t plane = (int64_t)p.batch * p.hkv * slab;
  const uint16_t* kb_hi = p.kbar + ((int64_t)b * p.hkv + g) * slab;
  const uint16_t* kb_lo = kb_hi + plane;
  const int nb = (n_wg + 31) / 32;

  // pooled-key operands of candidate block cb (B of the score product); a
  // wave loads a block while the products of the block before it run and
  // the statistics of the one before that are updated
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
  // scores of the loaded block for the 32 rows (log2 units)
  auto scores = [&]() -> f32x16_t {
    f32x16_t acc = {};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi[ks], kh[ks], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi[ks], kl[ks], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo[ks], kh[ks], acc, 0, 0, 0);
    }
    return acc;
  };
  // "have rowmax" flags as a bitmap per tile (in the radix histogram space,
  // which is free until the selection)
  uint32_t* sHrmBits = &sHist[0][0];   // [TPW][kMaxCandidates / 32]
  static_assert(TPW * (kMaxCandidates / 32) <= NWAVE * 256, "bitmap fits");
  for (int x = tid; x < TPW * (kMaxCandidates / 32); x += NT) sHrmBits[x] = 0u;

  // ---- 3) pass 1: per-row max, arg-max (lowest block) and sum, online
  RowStat st[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) st[r] = RowStat{kNegInf, 0.f, 0x7FFFFFFF};
  // software-pipelined: the products of block cb + NWAVE are issued before
  // the statistics of block cb, whose vector work then overlaps them, and
  // the operands of block cb + 2 NWAVE are loaded meanwhile (near the end
  // the index is clamped to the last block; that load goes unused)
  auto stats1 = [&](const f32x16_t& acc, int cb) {
    const int j = cb * 32 + col;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      // one exponential per element: exp2(-|s - m|) rescales the sum when s
      // raises the max (blocks arrive in ascending order per lane, so a
      // strict raise keeps the lowest block index) and is s's term otherwise
      const float s = acc[r];
      const float d = s - st[r].m;            // +inf while the row is empty
      const bool up = d > 0.f;
      const float e = __builtin_amdgcn_exp2f(up ? -d : d);
      const float zn = up ? fmaf(st[r].z, e, 1.f) : st[r].z + e;
      const bool valid = j < cand[r];
      st[r].z = valid ? zn : st[r].z;
      st[r].a = valid && up ? j : st[r].a;
      st[r].m = valid && up ? s : st[r].m;
    }
  };
  f32x16_t acc_cur = {};
  if (wave < nb) {
    load_ops(wave);
    acc_cur = scores();
    if (wave + NWAVE < nb) load_ops(wave + NWAVE);
  }
  int cb1 = wave;
  for (; cb1 + NWAVE < nb; cb1 += NWAVE) {
    const f32x16_t acc_next = scores();
    load_ops(min(cb1 + 2 * NWAVE, nb - 1));
    stats1(acc_cur, cb1);
    acc_cur = acc_next;
  }
  if (cb1 < nb) stats1(acc_cur, cb1);
  // merge the 128 partial statistics of every row (32 candidate lanes x
  // NWAVE waves): each lane puts its 16 rows' partials into LDS, then eight
  // threads per row merge 16 partials each (max first, then the sum rescaled
  // to it and the lowest block index reaching it) and combine over three
  // lane steps
  float* sPm = reinterpret_cast<float*>(sKeyRaw);
  float* sPz = sPm + 32 * kPartStride;
  int* sPa = reinterpret_cast<int*>(sPz + 32 * kPartStride);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int at = (8 * (r >> 2) + 4 * hf + (r & 3)) * kPartStride + wave * 32 + col;
    sPm[at] = st[r].m;
    sPz[at] = st[r].z;
    sPa[at] = st[r].a;
  }
  __syncthreads();
  {
    constexpr int PER = 32 * NWAVE / 8;
    const int row = tid >> 3;
    const int base = row * kPartStride + (tid & 7);
    float mx = kNegInf;
#pragma unroll
    for (int x = 0; x < PER; ++x) mx = fmaxf(mx, sPm[base + 8 * x]);
    RowStat s{mx, 0.f, 0x7FFFFFFF};
    if (mx != kNegInf) {
#pragma unroll
      for (int x = 0; x < PER; ++x) {
        const float mi = sPm[base + 8 * x];
        if (mi != kNegInf) s.z += sPz[base + 8 * x] * __builtin_amdgcn_exp2f(mi - mx);
        if (mi == mx) s.a = min(s.a, sPa[base + 8 * x]);
      }
    }
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) {
      RowStat o;
      o.m = __shfl_xor(s.m, off);
      o.z = __shfl_xor(s.z, off);
      o.a = __shfl_xor(s.a, off);
      s = merge(s, o);
    }
    if ((tid & 7) == 0) {
      sRowM[row] = s.m;
      sRowInvZ[row] = s.z > 0.f ? 1.f / s.z : 0.f;
      if (s.m != kNegInf && row < MR) {
        const int t = row / RPT;
        atomicOr(&sHrmBits[t * (kMaxCandidates / 32) + (s.a >> 5)], 1u << (s.a & 31));
      }
    }
  }
  __syncthreads();

  // ---- 4) pass 2: importance w and HRM flag per (tile, candidate) -> keys
  float rm[16], riz[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = 8 * (r >> 2) + 4 * hf + (r & 3);
    rm[r] = sRowM[m];
    riz[r] = sRowInvZ[m];
  }
  if (tid < TPW) sHrm[tid] = 0;
  __syncthreads();

  auto emit = [&](int t, int j, float wsum) {
    const int i = i0 + t;
    unsigned long long key = ~0ull;
    if (j < n_t[t]) {
      const float w = wsum / (float)rows_t[t];
      const bool hrm = (sHrmBits[t * (kMaxCandidates / 32) + (j >> 5)] >> (j & 31)) & 1u;
      if (hrm) atomicAdd(&sHrm[t], 1);
      const uint32_t wb = __float_as_uint(w);   // w >= 0: bit order == value order
      key = ((unsigned long long)(hrm ? 0u : 1u) << 63) |
            ((unsigned long long)(0x7FFFFFFFu - wb) << 32) | (uint32_t)j;
      const int64_t row = mrow0 + i;
      if (p.debug_w != nullptr) p.debug_w[row * p.n_max + j] = w;
      if (p.debug_hrm != nullptr) p.debug_hrm[row * p.n_max + j] = hrm ? 1 : 0;
    }
    sKey[t][j] = key;   // j < nb * 32 <= kMaxCandidates
  };

  // software-pipelined like pass 1
  auto weights = [&](const f32x16_t& acc, int cb) {
    const int j = cb * 32 + col;
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
    if (kShared) {
      // one tile: every row of the accumulator
      const float w = part[0] + part[1] + part[2] + part[3];
      const float wt = w + __shfl_xor(w, 32);
      if (hf == 0) emit(0, j, wt);
    } else if (R == 8) {
      // tile g4 = rows 8g4 .. 8g4+7: four in this lane, four in lane ^ 32
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const float w = part[g4] + __shfl_xor(part[g4], 32);
        if (hf == 0) emit(g4, j, w);
      }
    } else {
      // R == 4: tile 2*g4 + hf = rows 8g4 + 4hf .. +3, all in this lane
#pragma unroll
      for (int g4 = 0; g4 < 2; ++g4) emit(2 * g4 + hf, j, part[g4]);
    }
  };
  acc_cur = (f32x16_t){};
  if (wave < nb) {
    load_ops(wave);
    acc_cur = scores();
    if (wave + NWAVE < nb) load_ops(wave + NWAVE);
  }
  int cb2 = wave;
  for (; cb2 + NWAVE < nb; cb2 += NWAVE) {
    const f32x16_t acc_next = scores();
    load_ops(min(cb2 + 2 * NWAVE, nb - 1));
    weights(acc_cur, cb2);
    acc_cur = acc_next;
  }
  if (cb2 < nb) weights(acc_cur, cb2);
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
      for (int shift = 24; shift >= 0 && !top_bound; shift -= 8) {
        for (int bin = lane; bin < 256; bin += 64) sHist[t][bin] = 0;
#pragma unroll
        for (int e = 0; e < kPerLane; ++e) {
          if (64 * e >= n) break;
          if (lane + 64 * e < n && (hk[e] & pmask) == prefix)
            atomicAdd(&sHist[t][(hk[e] >> shift) & 255u], 1u);
        }
        uint32_t c[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) c[e] = sHist[t][4 * lane + e];
        const uint32_t mine = c[0] + c[1] + c[2] + c[3];
        uint32_t incl = mine;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const uint32_t o = __shfl_up(incl, off);
          if (lane >= off) incl += o;
        }
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
        const int src = __ffsll((long long)found) - 1;
        digit = __shfl(digit, src);
        need = __shfl(left, src);
        prefix |= (uint32_t)digit << shift;
        pmask |= 0xFFu << shift;
      }
      // compact keys with upper half <= prefix to the front, keeping order
      int written = 0;
      for (int base = 0; base < n; base += 64) {
        const int idx = base + lane;
        const unsigned long long key = idx < n ? sKey[t][idx] : ~0ull;
        const bool keep = idx < n && (uint32_t)(key >> 32) <= prefix;
        const unsigned long long bal = __ballot(keep);
        const int pos = written + __popcll(bal & ((1ull << lane) - 1ull));
        if (keep) sKey[t][pos] = key;
        written += __popcll(bal);
      }
      sel = written;
    }

    // ---- 6) bitonic sort of the kept keys, ascending, by this wavefront
    // alone (LDS operations of one wavefront complete in order, so a step
    // sees the writes of the step before it without a workgroup barrier)
    int npow = 1;
    while (npow < sel) npow <<= 1;
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

  // ---- 7) first k entries of every tile, remapped pages, counts
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int i = i0 + t;
    if (i >= p.nqb) break;
    const int64_t row = mrow0 + i;
    const int n = n_t[t];
    const int k = k_t[t];
    for (int s = tid; s < p.capacity; s += NT) {
      int blk = -1;
      if (s < k) blk = (int)(sKey[t][s] & 0xFFFFFFFFu);
      p.ordered_blocks[row * p.capacity + s] = blk;
      // the block's pages; -1 for a page past the sequence's end
      for (int e = 0; e < p.ppb; ++e) {
        int pg = -1;
        if (blk >= 0 && blk * kvb + e * kPage < L) pg = pt[blk * p.ppb + e];
        p.ordered_pages[(row * p.capacity + s) * p.ppb + e] = pg;
      }
    }
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
    hipLaunchKernelGGL((kap_pool_keys<D>), dim3(nkb, p.batch), dim3(256), 0, stream, p);
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
