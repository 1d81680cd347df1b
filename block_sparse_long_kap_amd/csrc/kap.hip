// Kernel-Aware Proxy (KAP) for gfx950: block-pooled scoring, "have rowmax"
// flags, flag-grouped ordering and stage-1 budget truncation.
//
// Method: CoSA (paper text on paperpeel.com), §4.2 "Kernel-Aware Proxy
// Design" with App. C.1 "Illustrative KAP Ordering": every candidate key
// block of a query block receives an importance score and an HRM flag; the
// HRM and non-HRM groups are sorted independently by score, the HRM group is
// placed first and the leading entries under the stage-1 budget form the
// ordered mask M_KAP.  §5.1 ("Implementation details") fuses scoring and
// pooling into one kernel to keep the proxy cheap.  The body of "Block
// ranking" is not in the text; the score used here is the block-pooled logit
// (mean query of 16 consecutive rows against the mean key of a page), its
// per-proxy-row softmax averaged over the tile's proxy rows, and HRM marks
// the arg-max block of each proxy row.
//
// Two launches:
//   kap_pool_keys   one workgroup per (sequence, key block): streams the
//                   page of every KV head once from HBM and writes the fp32
//                   mean key, d-major ([d][block]) so the scoring loads of
//                   neighbouring candidates are contiguous.
//   kap_select      one workgroup per mask row (sequence, query head, tile):
//                   pools the tile's queries from HBM into LDS, scores up to
//                   2048 candidates in registers (fp32 FMA), reduces the
//                   per-proxy-row max / arg-max / sum with wavefront
//                   reductions, builds 64-bit sort keys (not HRM, -w, j),
//                   bitonic-sorts them in LDS and writes the first k block
//                   ids together with their remapped pages.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cosa_internal.h"

namespace cosa {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---------------------------------------------------------------------------
// Key pooling: kbar[b][g][d][j] = mean of the valid keys of block j.
template <int D>
__global__ __launch_bounds__(256) void kap_pool_keys(const KapParams p) {
  constexpr int NT = 256;
  constexpr int KCH = D / 8;          // 16-byte chunks per key row
  constexpr int RG = NT / KCH;        // row groups
  __shared__ float red[RG][D];

  const int j = blockIdx.x;
  const int b = blockIdx.y;
  const int q0 = p.cu_seqlens[b];
  const int L = p.cu_seqlens[b + 1] - q0;
  if (j * kPage >= L) return;
  const int nvalid = min(kPage, L - j * kPage);
  const int page = p.page_table[(int64_t)b * p.max_pages + j];
  const int tid = threadIdx.x;
  const int c = tid % KCH;
  const int rg = tid / KCH;
  const float inv = 1.f / (float)nvalid;

  for (int g = 0; g < p.hkv; ++g) {
    const uint16_t* base = p.k_pool + ((int64_t)page * p.hkv + g) * (kPage * D) + c * 8;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    for (int r = rg; r < nvalid; r += RG) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(base + r * D);
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
      p.kbar[(((int64_t)b * p.hkv + g) * D + tid) * p.n_max + j] = sum * inv;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Wavefront arg-max (ties to the lowest index) and sum.
__device__ __forceinline__ void wave_argmax(float& v, int& idx) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(v, off);
    const int oi = __shfl_xor(idx, off);
    if (ov > v || (ov == v && oi < idx)) {
      v = ov;
      idx = oi;
    }
  }
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

template <int D, int R>
__global__ __launch_bounds__(256) void kap_select(const KapParams p) {
  constexpr int NT = 256;
  constexpr int NWAVE = NT / 64;
  constexpr int M = kMaxCandidates / NT;     // candidates per thread
  constexpr int BQ = R * kProxyRows;
  constexpr int D4 = D / 4;

  __shared__ __attribute__((aligned(16))) float sQ[R][D];
  __shared__ unsigned long long sKey[kMaxCandidates];
  __shared__ float sRedV[NWAVE][R];
  __shared__ int sRedI[NWAVE][R];
  __shared__ float sRowMax[R];
  __shared__ int sRowArg[R];
  __shared__ float sRowSum[R];
  __shared__ int sCount[NWAVE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // Same longest-first order as the attention kernel (no XCD affinity needed).
  const int per_level = p.batch * p.hq;
  const int level = blockIdx.x / per_level;
  const int rem = blockIdx.x - level * per_level;
  const int b = rem / p.hq;
  const int h = rem - b * p.hq;
  const int i = p.nqb - 1 - level;
  const int g = h / (p.hq / p.hkv);
  const int64_t row = ((int64_t)b * p.hq + h) * p.nqb + i;
  const int q0 = p.cu_seqlens[b];
  const int L = p.cu_seqlens[b + 1] - q0;
  const int tile_q0 = i * BQ;
  int32_t* ob = p.ordered_blocks + row * p.capacity;
  int32_t* opg = p.ordered_pages + row * p.capacity;

  if (tile_q0 >= L) {
    for (int t = tid; t < p.capacity; t += NT) {
      ob[t] = -1;
      opg[t] = -1;
    }
    if (tid == 0) {
      p.counts[row] = 0;
      if (p.hrm_counts != nullptr) p.hrm_counts[row] = 0;
    }
    if (p.debug_w != nullptr)
      for (int jj = tid; jj < p.n_max; jj += NT) p.debug_w[row * p.n_max + jj] = 0.f;
    if (p.debug_hrm != nullptr)
      for (int jj = tid; jj < p.n_max; jj += NT) p.debug_hrm[row * p.n_max + jj] = 0;
    return;
  }

  // ---- proxy rows: mean of 16 consecutive valid queries, pre-scaled
  for (int idx = tid; idx < R * D4; idx += NT) {
    const int r = idx / D4, d4 = idx - r * D4;
    const int a = tile_q0 + r * kProxyRows;
    const int e = min(a + kProxyRows, L);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int t = a; t < e; ++t) {
      const u32x2_t v =
          *reinterpret_cast<const u32x2_t*>(p.q + ((int64_t)(q0 + t) * p.hq + h) * D + 4 * d4);
      acc[0] += bf16_lo(v[0]);
      acc[1] += bf16_hi(v[0]);
      acc[2] += bf16_lo(v[1]);
      acc[3] += bf16_hi(v[1]);
    }
    const float f = e > a ? p.scale / (float)(e - a) : 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) sQ[r][4 * d4 + k] = acc[k] * f;
  }
  // per proxy row: last valid position -> candidate count (0 if the row is empty)
  int rcand[R];
  int nrows = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int a = tile_q0 + r * kProxyRows;
    const int last = min(a + kProxyRows, L) - 1;
    rcand[r] = a < L ? last / kPage + 1 : 0;
    nrows += a < L ? 1 : 0;
  }
  const int n = (min(tile_q0 + BQ, L) - 1) / kPage + 1;   // tile candidates
  __syncthreads();

  // ---- scores s[r][j] for the thread's candidates j = tid + NT*m
  float s[M][R];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r) s[m][r] = 0.f;
  const float* kb = p.kbar + ((int64_t)b * p.hkv + g) * D * p.n_max;
  for (int d4 = 0; d4 < D4; ++d4) {
    float qv[R][4];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int k = 0; k < 4; ++k) qv[r][k] = sQ[r][4 * d4 + k];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int j = tid + NT * m;
      if (j < n) {
        float kv[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) kv[k] = kb[(int64_t)(4 * d4 + k) * p.n_max + j];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int k = 0; k < 4; ++k) s[m][r] = fmaf(qv[r][k], kv[k], s[m][r]);
      }
    }
  }

  // ---- per proxy row: max and arg-max over its candidates
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float v = kNegInf;
    int idx = 0x7FFFFFFF;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int j = tid + NT * m;
      if (j < rcand[r] && s[m][r] > v) {   // ascending j per thread: strict > keeps lowest
        v = s[m][r];
        idx = j;
      }
    }
    wave_argmax(v, idx);
    if (lane == 0) {
      sRedV[wave][r] = v;
      sRedI[wave][r] = idx;
    }
  }
  __syncthreads();
  if (tid < R) {
    float v = sRedV[0][tid];
    int idx = sRedI[0][tid];
    for (int w = 1; w < NWAVE; ++w) {
      const float ov = sRedV[w][tid];
      const int oi = sRedI[w][tid];
      if (ov > v || (ov == v && oi < idx)) {
        v = ov;
        idx = oi;
      }
    }
    sRowMax[tid] = v;
    sRowArg[tid] = idx;
  }
  __syncthreads();

  // ---- exponentials and per-row sums
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float mx = sRowMax[r];
    float part = 0.f;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int j = tid + NT * m;
      const float e = j < rcand[r] ? expf(s[m][r] - mx) : 0.f;
      s[m][r] = e;
      part += e;
    }
    part = wave_sum(part);
    if (lane == 0) sRedV[wave][r] = part;
  }
  __syncthreads();
  if (tid < R) {
    float sum = 0.f;
    for (int w = 0; w < NWAVE; ++w) sum += sRedV[w][tid];
    sRowSum[tid] = sum;
  }
  __syncthreads();

  // ---- importance, HRM flag and sort key per candidate
  float inv_sum[R];
#pragma unroll
  for (int r = 0; r < R; ++r) inv_sum[r] = rcand[r] > 0 ? 1.f / sRowSum[r] : 0.f;
  const float inv_rows = 1.f / (float)nrows;
  int my_hrm = 0;
  int npow = 1;
  while (npow < n) npow <<= 1;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int j = tid + NT * m;
    if (j < npow) {
      unsigned long long key = ~0ull;
      if (j < n) {
        float w = 0.f;
        bool hrm = false;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          w += s[m][r] * inv_sum[r];
          hrm |= (rcand[r] > 0 && sRowArg[r] == j);
        }
        w *= inv_rows;
        my_hrm += hrm ? 1 : 0;
        const uint32_t wb = __float_as_uint(w);   // w >= 0: bit order == value order
        key = ((unsigned long long)(hrm ? 0u : 1u) << 63) |
              ((unsigned long long)(0x7FFFFFFFu - wb) << 32) | (uint32_t)j;
        if (p.debug_w != nullptr) p.debug_w[row * p.n_max + j] = w;
        if (p.debug_hrm != nullptr) p.debug_hrm[row * p.n_max + j] = hrm ? 1 : 0;
      }
      sKey[j] = key;
    }
  }
  if (p.debug_w != nullptr)
    for (int jj = n + tid; jj < p.n_max; jj += NT) p.debug_w[row * p.n_max + jj] = 0.f;
  if (p.debug_hrm != nullptr)
    for (int jj = n + tid; jj < p.n_max; jj += NT) p.debug_hrm[row * p.n_max + jj] = 0;
  {
    int c = my_hrm;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off);
    if (lane == 0) sCount[wave] = c;
  }
  __syncthreads();

  // ---- bitonic sort of npow keys, ascending
  for (int size = 2; size <= npow; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int pi = tid; pi < (npow >> 1); pi += NT) {
        const int lo = 2 * stride * (pi / stride) + (pi % stride);
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const unsigned long long a = sKey[lo], c = sKey[hi];
        if ((a > c) == up) {
          sKey[lo] = c;
          sKey[hi] = a;
        }
      }
      __syncthreads();
    }
  }

  // ---- first k entries in order, remapped pages, counts
  const long long kk = ((long long)n * p.beta_ppm + 999999) / 1000000;
  const int k = (int)(kk < 1 ? 1 : (kk > n ? n : kk));
  const int32_t* pt = p.page_table + (int64_t)b * p.max_pages;
  for (int t = tid; t < p.capacity; t += NT) {
    int blk = -1, pg = -1;
    if (t < k) {
      blk = (int)(sKey[t] & 0xFFFFFFFFu);
      pg = pt[blk];
    }
    ob[t] = blk;
    opg[t] = pg;
  }
  if (tid == 0) {
    int nh = 0;
    for (int w = 0; w < NWAVE; ++w) nh += sCount[w];
    p.counts[row] = k;
    if (p.hrm_counts != nullptr) p.hrm_counts[row] = nh < k ? nh : k;
  }
}

template <int D, int R>
hipError_t launch_kap_t(const KapParams& p, hipStream_t stream) {
  const int nkb = p.n_max;
  if (p.batch <= 0 || nkb <= 0) return hipSuccess;
  hipLaunchKernelGGL((kap_pool_keys<D>), dim3(nkb, p.batch), dim3(256), 0, stream, p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t grid = (int64_t)p.batch * p.hq * p.nqb;
  hipLaunchKernelGGL((kap_select<D, R>), dim3((unsigned)grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kap(const KapParams& p, int head_dim, int q_block, hipStream_t stream) {
  if (head_dim == 128 && q_block == 128) return launch_kap_t<128, 8>(p, stream);
  if (head_dim == 128 && q_block == 64) return launch_kap_t<128, 4>(p, stream);
  if (head_dim == 64 && q_block == 128) return launch_kap_t<64, 8>(p, stream);
  if (head_dim == 64 && q_block == 64) return launch_kap_t<64, 4>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace cosa
