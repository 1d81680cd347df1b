// Paged causal prefill attention for gfx950: the Ordered-Skipping Kernel and
// the dense baseline share this one kernel template.
//
// Method: CoSA (paper text on paperpeel.com), §4.3 "Ordered-Skipping Kernel":
// the kernel follows the computation-order mask by remapping pages of the
// paged KV cache (it jumps to each physical page, in any order) and applies the
// in-kernel skip of §3.3 Eq. (5) at the granularity of one query tile
// (App. D.1: one tile-wide vote combined from the row-wise predicates, made
// from the on-chip online-softmax maxima with no extra logits and no extra
// global-memory traffic).  Dense mode walks every causal block in ascending
// order through the page table and never votes.  Logical mode walks the same
// blocks but computes only those selected by a block bitmask, paying the loop
// and the per-block barrier on the others (the logical mask skipping that
// App. D.3 / Fig. B compares physical page jumping against).
//
// gfx950 mapping (one workgroup = one query tile of one query head, or of
// two query heads of a KV group on the dense walk, which then share every K
// and V page the workgroup loads):
//   * NW wavefronts of 64 lanes per head, 32 query rows per wavefront
//     (tile = 32*NW).
//   * Logits are formed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: each lane then owns one query column and 32
//     of the 64 keys of a page, so the row max is an in-register reduction
//     plus one exchange with the partner lane (lane ^ 32).
//   * The value product is O^T = V^T P^T on the same MFMA: P^T comes straight
//     from the S^T accumulator registers (rounded to bf16); the V^T operand
//     is read from the page as stored ([key][D]) with the gfx950 transposing
//     LDS read (ds_read_b64_tr_b16), in the key order the accumulator layout
//     implies.
//   * K and V pages are copied from HBM straight into LDS (no registers)
//     through a ring of NS stages: K NS pages ahead, V NS - 1 ahead (NS = 2
//     with two workgroups per CU; NS = 4 for the two-head workgroup, alone on
//     its CU).  One workgroup barrier per visited page carries both the LDS
//     hand-off and the tile-wide skip vote; before it each wavefront waits
//     only for its copies of the pages the next steps read.
//   * Tile order: one (sequence, KV head) group at a time over the whole
//     chip, longest tiles (most causal blocks) first inside the group, so the
//     working set is that group's pages.  A level-major order and one that
//     pins each group to one XCD are kept as alternatives.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "cosa_internal.h"

// Two query heads of a KV group per workgroup on the dense walk (0 turns the
// pairing off).
#ifndef COSA_HEAD_PAIRS
#define COSA_HEAD_PAIRS 1
#endif
// Dense walk: the two heads of a workgroup in opposite phases (the products
// of one head beside the softmax of the other); 0 selects the kernel whose
// two heads run each page step together.
#ifndef COSA_DENSE_PP
#define COSA_DENSE_PP 1
#endif

namespace cosa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;
// Last word of a raw (untyped) buffer resource on CDNA: 32-bit data format,
// no swizzle, no index stride.
constexpr int kBufferWord3 = 0x00020000;

// The two 32-lane halves of a wavefront exchanged in one VALU instruction
// (v_permlane32_swap): one of the returned values is the lane's own, the
// other its partner's (lane ^ 32), so symmetric combinations need no order.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// K and V pages in LDS: [64 keys][D] bf16 as in HBM, with the 16-byte
// chunks of each row permuted by a function of the row.  Pages are copied
// HBM -> LDS directly (no registers): lane i of a copy instruction writes the
// i-th 16-byte slot of its wavefront's span and fetches whichever logical
// chunk belongs in that slot.  The permutation (swap of the two 2-bit halves
// of row mod 16, for D = 128) spreads both access patterns over the banks:
// the QK operand reads (32 consecutive rows, one chunk) and the transposed
// P V operand reads (8 rows x 4 chunks per instruction).
template <int D>
struct PageLayout {
  static constexpr int kChunks = D / 8;
  static constexpr int kBytes = kPage * D * 2;
  static __device__ __forceinline__ int swz(int row) {
    if constexpr (kChunks >= 16)
      return ((row & 3) << 2) | ((row >> 2) & 3);
    else
      return ((row & 3) << 1) | ((row >> 2) & 1);
  }
  static __device__ __forceinline__ int offset(int row, int chunk16) {
    return row * (D * 2) + ((chunk16 ^ swz(row)) << 4);
  }
};

// Decode the workgroup's (sequence, head unit, tile).  A head unit is HP
// consecutive query heads of one KV group; hq_u = Hq / HP units per sequence.
// Every order launches the tiles with more causal blocks first
// (longest-processing-time first).
__device__ __forceinline__ void decode_tile(const AttnParams& p, int bid, int hq_u, int& b, int& h,
                                            int& i) {
  const int hg = hq_u / p.hkv;
  if (p.order == kOrderXcdGroup) {
    // consecutive workgroup ids go round-robin over the 8 XCDs: pin each
    // (sequence, KV head) group to one XCD so its pages stay in that L2
    const int x = bid & 7;
    const int r = bid >> 3;
    const int groups_per_xcd = p.xcd_groups >> 3;
    const int per_level = groups_per_xcd * hg;
    const int level = r / per_level;
    const int rem = r - level * per_level;
    const int gi = rem / hg;
    const int hh = rem - gi * hg;
    const int G = x + 8 * gi;
    b = G / p.hkv;
    const int g = G - b * p.hkv;
    h = g * hg + hh;
    i = p.nqb - 1 - level;
  } else if (p.order == kOrderGroupXcd) {
    // group-major sequence of (group, level) units, each unit's head units on
    // one XCD (workgroup ids go round-robin over the 8 XCDs): unit u runs on
    // XCD u % 8, each XCD takes its units in sequence order, so the heads of
    // a tile, whose kept pages overlap, share that XCD's L2
    const int x = bid & 7;
    const int r = bid >> 3;
    const int unit = (r / hg) * 8 + x;
    const int hh = r - (r / hg) * hg;
    const int gl = unit / p.nqb;   // group within the launched range
    const int G = p.group_begin + gl;
    const int level = unit - gl * p.nqb;
    b = G / p.hkv;
    const int g = G - b * p.hkv;
    h = g * hg + hh;
    i = p.nqb - 1 - level;
  } else if (p.order == kOrderGroupMajor) {
    // one (sequence, KV head) group at a time over the whole chip, so the
    // working set is that group's pages (64 MB at 128K) and repeated page
    // visits across tiles and query heads hit the memory-side cache
    const int per_group = hg * p.nqb;
    const int local = bid / per_group;
    const int G = p.group_begin + local;
    const int r = bid - local * per_group;
    const int level = r / hg;
    const int hh = r - level * hg;
    b = G / p.hkv;
    const int g = G - b * p.hkv;
    h = g * hg + hh;
    i = p.nqb - 1 - level;
  } else {
    const int per_level = p.batch * hq_u;
    const int level = bid / per_level;
    const int rem = bid - level * per_level;
    b = rem / hq_u;
    h = rem - b * hq_u;
    i = p.nqb - 1 - level;
  }
}

// s_waitcnt on the vector-memory count alone (export and LDS counts left at
// their maxima): at most N of this wavefront's vector memory operations stay
// outstanding.  They complete in issue order.
template <int N>
__device__ __forceinline__ void wait_vm_c() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0xF70);
}

// Workgroup barrier that orders LDS accesses (wait for this wavefront's LDS
// operations, then s_barrier) but, unlike __syncthreads(), does not also wait
// for the wavefront's HBM -> LDS copies still in flight; the memory clobber
// keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Template parameters: D head dim; NW wavefronts per query head, 32 query
// rows each (the tile is 32 NW rows of one head); kMode the page walk; PPB
// pages per logical key block (1: a 64-key block is one page; 2: a 128-key
// block is resolved through two pages, with one decision per block, and each
// 32 rows are taken by a pair of wavefronts, one page each); HP query
// heads per workgroup (2: two query heads of one KV group that walk the same
// page list, dense or a mask shared by the KV group, compute on every K and V
// page the workgroup loads, which halves the page traffic per query row); NS
// LDS stages per operand (copies run NS blocks ahead for K and NS - 1 for V).
// Occupancy: two workgroups per CU (64 KB of LDS each) give two wavefronts
// per SIMD for 4-wavefront tiles; 2-wavefront tiles (64 rows) get one per
// SIMD however many fit, so they ask for one and may use the whole file.
// Two-page blocks (128 KB of LDS, one workgroup per CU) get their second
// wavefront per SIMD from the pairs.
template <int D, int NW, int kMode, int PPB, int HP, int NS>
__global__ __launch_bounds__(NW * (PPB == 2 ? 2 : HP) * 64,
                             (PPB == 1 && HP == 1 && NW >= 4) ? 2 : 1) void
attn_fwd_kernel(const AttnParams p) {
  constexpr bool kOrdered = kMode == kModeOrdered;
  constexpr bool kLogical = kMode == kModeLogical;
  static_assert(PPB == 1 || PPB == 2, "one or two pages per logical block");
  static_assert(HP == 1 || HP == 2, "one or two query heads per workgroup");
  static_assert(NS == 2 || NS == 4, "two or four LDS stages");
  static_assert(NS * PPB <= 4, "at most four LDS page buffers per operand");
  static_assert(HP == 1 || !kLogical, "logical skipping walks one head per workgroup");
  constexpr int KVB = kPage * PPB;                   // keys per logical block
  constexpr int MB = 2 * PPB;                        // 32-key S^T blocks per logical block
  // Two-page blocks: the two wavefronts of a pair take the same 32 query rows
  // and one page of the block each (twice the wavefronts per workgroup, one
  // page of products each), vote on their own page and share their row
  // maxima, so that both keep the same running max; their partial outputs
  // are added at the end.
  constexpr bool kPair = PPB == 2;
  constexpr int NGRP = kPair ? 2 : HP;               // groups of NW wavefronts
  constexpr int MBW = kPair ? 2 : MB;                // S^T blocks per wavefront and step
  constexpr int NWT = NW * NGRP;                     // wavefronts per workgroup
  constexpr int NT = NWT * 64;
  constexpr int NTH = NW * 64;                       // threads per head
  constexpr int BQ = NW * 32;                        // query rows per head (the tile)
  constexpr int KCH = D / 8;                         // 16-byte chunks per key row
  constexpr int K_TOTAL = kPage * KCH;               // 16-byte chunks per page
  static_assert(K_TOTAL % NT == 0, "page copy must split evenly over the workgroup");
  constexpr int K_PER = K_TOTAL / NT;
  static_assert(NS == 2 || PPB == 1, "four stages hold one-page blocks");
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;
  // Lazy rescaling: the reference max used for the exponentials only moves
  // when the true running max exceeds it by more than 2^kRescale, so the
  // accumulator is rarely rescaled; weights stay <= 2^kRescale.
  constexpr float kRescale = 8.f;

  // Page buffers per operand as distinct LDS objects, so that the compiler
  // can tell reads of one buffer from the asynchronous HBM->LDS copies into
  // another and does not wait for those copies before the reads.
  // Buffer stage * PPB + s holds page s of the logical block of that stage.
  constexpr int kNB = NS * PPB;
  constexpr int kXtra = kNB == 4 ? PageLayout<D>::kBytes : 16;
  __shared__ __attribute__((aligned(16))) unsigned char sK0[PageLayout<D>::kBytes];
  __shared__ __attribute__((aligned(16))) unsigned char sK1[PageLayout<D>::kBytes];
  __shared__ __attribute__((aligned(16))) unsigned char sK2[kXtra];
  __shared__ __attribute__((aligned(16))) unsigned char sK3[kXtra];
  __shared__ __attribute__((aligned(16))) unsigned char sV0[PageLayout<D>::kBytes];
  __shared__ __attribute__((aligned(16))) unsigned char sV1[PageLayout<D>::kBytes];
  __shared__ __attribute__((aligned(16))) unsigned char sV2[kXtra];
  __shared__ __attribute__((aligned(16))) unsigned char sV3[kXtra];
  __shared__ int sVote[2][NWT];
  // two-page blocks: each page half's block row maxima, per vote buffer
  __shared__ float sBm[2][2][kPair ? NW * 32 : 1];
  __shared__ int sSlotP[2][64 * PPB];   // [ring chunk][slot * PPB + page]
  __shared__ int sSlotB[2][64];         // [ring chunk][slot]: logical block
  // logical-skip mode: the tile's block bitmask (up to 16384 causal blocks)
  __shared__ uint32_t sBits[kLogical ? 512 : 1];
  // ordered mode: each head's skip decisions, one bit per slot (up to 16384)
  __shared__ uint32_t sRec[kOrdered ? HP : 1][kOrdered ? 512 : 1];
  auto kbuf = [&](int stage, int s) -> unsigned char* {
    const int x = stage * PPB + s;
    return x == 0 ? sK0 : x == 1 ? sK1 : x == 2 ? sK2 : sK3;
  };
  auto vbuf_of = [&](int stage, int s) -> unsigned char* {
    const int x = stage * PPB + s;
    return x == 0 ? sV0 : x == 1 ? sV1 : x == 2 ? sV2 : sV3;
  };
  auto kraw = [&](int x) -> unsigned char* {
    return x == 0 ? sK0 : x == 1 ? sK1 : x == 2 ? sK2 : sK3;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // uniform by construction; telling the compiler keeps the LDS destinations
  // of the page copies and the head selection in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave / NW;                         // group of NW wavefronts
  const int hs = kPair ? 0 : grp;                    // head of the workgroup's unit
  const int ph = kPair ? grp : 0;                    // two-page blocks: this wavefront's page
  const int wv = wave - grp * NW;                    // wavefront within the tile
  const int tid_h = tid - grp * NTH;                 // thread within the group
  const bool head_writer = tid_h == 0 && ph == 0;
  const int hf = lane >> 5;
  const int col = lane & 31;

  int b, hu, i;
  decode_tile(p, blockIdx.x, p.hq / HP, b, hu, i);
  const int hg = p.hq / p.hkv;
  const int h = hu * HP + hs;
  const int g = (hu * HP) / hg;
  const int q0 = p.cu_seqlens[b];
  const int L = p.cu_seqlens[b + 1] - q0;
  const int tile_q0 = i * BQ;
  const int64_t row = ((int64_t)b * p.hq + h) * p.nqb + i;
  if (tile_q0 >= L) {
    if (kOrdered && p.row_stats != nullptr && head_writer) {
      p.row_stats[2 * row] = 0;
      p.row_stats[2 * row + 1] = 0;
    }
    return;
  }
  const int tile_last = min(tile_q0 + BQ, L) - 1;
  // mask row: per query head, or per KV head when the group shares its mask
  // (the host pairs heads only when they share the mask row, so the slot
  // count and the page walk are the same for the whole workgroup)
  const int64_t mrow =
      kOrdered ? ((int64_t)b * p.mask_heads + h / (p.hq / p.mask_heads)) * p.nqb + i : row;
  const int cnt = kOrdered ? p.counts[mrow] : tile_last / KVB + 1;
  if (kLogical) {
    const uint32_t* bits = p.block_mask + row * p.mask_words;
    for (int wd = tid; wd < (cnt + 31) / 32; wd += NT) sBits[wd] = bits[wd];
  }
  // logical-skip mode: is causal block t selected (uniform)
  auto selected = [&](int t) -> bool {
    if constexpr (kLogical)
      return (__builtin_amdgcn_readfirstlane(sBits[t >> 5]) >> (t & 31)) & 1u;
    else
      return true;
  };
  // read-only for the whole kernel: lets the uniform slot lookups go
  // through scalar loads instead of vector loads plus a vmcnt wait
  const int32_t* __restrict__ ob = kOrdered ? p.ordered_blocks + mrow * p.capacity : nullptr;
  const int32_t* __restrict__ op =
      kOrdered ? p.ordered_pages + mrow * p.capacity * PPB : nullptr;
  const int32_t* __restrict__ pt = p.page_table + (int64_t)b * p.max_pages;

  const int wave_q0 = tile_q0 + wv * 32;
  const int wave_last = min(wave_q0 + 31, L - 1);
  const int qpos = wave_q0 + col;
  const bool row_valid = qpos < L;
  const bool wave_has_rows = wave_q0 < L;

  // ---- Q^T operand (B of S^T = K Q^T), kept in registers for the whole tile
  bf16x8_t qf[KSTEPS];
  {
    const uint16_t* qp = p.q + ((int64_t)(q0 + qpos) * p.hq + h) * D + hf * 8;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (row_valid) v = *reinterpret_cast<const u32x4_t*>(qp + ks * 16);
      qf[ks] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // Slot -> (logical block, page) lookups come from a two-chunk ring of 64
  // entries in LDS (uniform-address reads, no vector-memory wait on the page
  // loop).  When slot 64c starts, wave 0 copies chunk c+1 from memory straight
  // into the ring half that chunk c-1 used (HBM -> LDS); it is read at least
  // 64 - NS slots and as many barriers later.
  // page entries: slot t's pages at page_src[t * PPB + s] (the ordered
  // mask's page list, or the page table, whose logical block t spans pages
  // t * PPB .. t * PPB + PPB - 1)
  const int32_t* __restrict__ page_src = kOrdered ? op : pt;
  if (wave == 0) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int e = 0; e < PPB; ++e) {
        const int x = c * 64 * PPB + e * 64 + lane;
        sSlotP[c][e * 64 + lane] = x < cnt * PPB ? page_src[x] : 0;
      }
      if (kOrdered) {
        const int t = c * 64 + lane;
        sSlotB[c][lane] = t < cnt ? ob[t] : 0;
      }
    }
  }
  __syncthreads();   // every wave reads the ring (and bitmask) just filled
  auto slot_page = [&](int t, int s) -> int {
    return __builtin_amdgcn_readfirstlane(sSlotP[(t >> 6) & 1][(t & 63) * PPB + s]);
  };
  auto slot_block = [&](int t) -> int {
    return kOrdered ? __builtin_amdgcn_readfirstlane(sSlotB[(t >> 6) & 1][t & 63]) : t;
  };
  auto advance_chunks = [&](int t_next) {
    if (wave == 0 && (t_next & 63) == 0 && t_next > 0 && ((t_next >> 6) + 1) * 64 < cnt) {
      const int c = (t_next >> 6) + 1;
#pragma unroll
      for (int e = 0; e < PPB; ++e) {
        // lanes past the count re-read a valid entry
        const int x = min(c * 64 * PPB + e * 64 + lane, cnt * PPB - 1);
        __builtin_amdgcn_global_load_lds(
            static_cast<const void*>(page_src + x),
            (__attribute__((address_space(3))) void*)&sSlotP[c & 1][e * 64], 4, 0, 0);
      }
      const int t = min(c * 64 + lane, cnt - 1);
      if (kOrdered)
        __builtin_amdgcn_global_load_lds(
            static_cast<const void*>(ob + t),
            (__attribute__((address_space(3))) void*)&sSlotB[c & 1][0], 4, 0, 0);
      // once per 64 slots: the ring copy lands before this wave reaches the
      // next barrier (and so before any wave reads the chunk)
      __builtin_amdgcn_s_waitcnt(0);
    }
  };
  const int64_t head_stride = (int64_t)kPage * D;              // elements per (page, head)
  const int64_t page_stride = (int64_t)p.hkv * head_stride;

  // ---- K and V pages: HBM -> LDS without registers (16 bytes per lane per
  // instruction).  Lane byte offsets inside a page are fixed for the kernel;
  // the page's base is uniform.
  uint32_t coff[K_PER];
#pragma unroll
  for (int e = 0; e < K_PER; ++e) {
    const int f = e * NT + tid;                // physical 16-byte slot in the page
    const int r = f / KCH;
    const int c = (f % KCH) ^ PageLayout<D>::swz(r);
    coff[e] = (uint32_t)(r * D + c * 8) * 2u;
  }
  // One buffer resource per (page, head) slice, built in scalar registers;
  // the lane offsets stay in the same VGPRs for the whole kernel.
  constexpr int kSliceBytes = kPage * D * 2;
  auto copy_page = [&](const uint16_t* pool, int page, unsigned char* dst) {
    const uint16_t* base = pool + (int64_t)page * page_stride + (int64_t)g * head_stride;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(base), (short)0, kSliceBytes, kBufferWord3);
#pragma unroll
    for (int e = 0; e < K_PER; ++e) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(dst + (e * NT + wave * 64) * 16), 16,
          (int)coff[e], 0, 0, 0);
    }
  };
  // the pages of slot t's logical block j that hold keys of the sequence;
  // returns the number of copy instructions this wavefront issued
  auto copy_k = [&](int t, int j, int stage) -> int {
    int n = 0;
#pragma unroll
    for (int s = 0; s < PPB; ++s)
      if (s == 0 || j * KVB + s * kPage < L) {
        copy_page(p.k_pool, slot_page(t, s), kbuf(stage, s));
        n += K_PER;
      }
    return n;
  };
  auto copy_v = [&](int t, int j, int stage) -> int {
    int n = 0;
#pragma unroll
    for (int s = 0; s < PPB; ++s)
      if (s == 0 || j * KVB + s * kPage < L) {
        copy_page(p.v_pool, slot_page(t, s), vbuf_of(stage, s));
        n += K_PER;
      }
    return n;
  };
  // The ring entries of a slot whose pages a later part of the step copies,
  // read ahead into registers (uniform values) so that the copies do not wait
  // for an LDS round trip after the barrier.  Any slot index maps inside the
  // ring (entries past the count are stale and unused).
  struct SlotRef {
    int page[PPB];
    int block;
  };
  auto slot_ref = [&](int t) -> SlotRef {
    SlotRef r;
#pragma unroll
    for (int s = 0; s < PPB; ++s) r.page[s] = sSlotP[(t >> 6) & 1][(t & 63) * PPB + s];
    r.block = (kOrdered && PPB > 1) ? sSlotB[(t >> 6) & 1][t & 63] : t;
    return r;
  };
  auto copy_ref = [&](const uint16_t* pool, const SlotRef& r, int stage, bool is_k) {
    const int j = __builtin_amdgcn_readfirstlane(r.block);
#pragma unroll
    for (int s = 0; s < PPB; ++s)
      if (s == 0 || j * KVB + s * kPage < L)
        copy_page(pool, __builtin_amdgcn_readfirstlane(r.page[s]),
                  is_k ? kbuf(stage, s) : vbuf_of(stage, s));
  };

  f32x16_t o[DBLK];
#pragma unroll
  for (int md = 0; md < DBLK; ++md) o[md] = (f32x16_t){};
  float m_true = kNegInf;   // running max of this lane's query row (log2 units)
  float m_ref = kNegInf;    // reference max of the exponentials (<= m_true)
  float lsum = 0.f;         // this lane's half of the running sum, relative to m_ref
  int nskip = 0;
  bool v_have = true;       // the V page(s) of the current slot were prefetched
  uint32_t rec_word = 0;    // skip bits of the head's current 32 slots
  const bool skip_on = kOrdered && p.skip_mode != kSkipOff;
  // threshold in log2 units: fixed, or log2(L / Delta) for this sequence
  const float tau_l2 = p.skip_mode == kSkipDelta ? __log2f((float)L) - p.log2_delta : p.tau_log2;
  const float c2 = p.scale_log2;

  // ---- building blocks of one page step (all straight-line code, so that
  // the compiler can interleave them inside one basic block)
  // S^T(block) = K Q^T for this wave's 32 queries: raw dot products; S^T
  // block mb holds keys 32mb.. of the logical block (page mb / 2).  The K
  // operand reads run two k-steps ahead of the products (one with two heads
  // per workgroup, whose wavefronts hold more state).
  auto qk = [&](int stage, f32x16_t (&sacc)[MBW]) {
    constexpr int kAhead = HP == 1 ? 2 : 1;
    u32x4_t a[kAhead + 1][MBW];
    auto load = [&](int ks) {
#pragma unroll
      for (int mb = 0; mb < MBW; ++mb)
        a[ks % (kAhead + 1)][mb] = *reinterpret_cast<const u32x4_t*>(
            kbuf(stage, kPair ? ph : mb >> 1) +
            PageLayout<D>::offset((mb & 1) * 32 + col, 2 * ks + hf));
    };
#pragma unroll
    for (int ks = 0; ks < kAhead && ks < KSTEPS; ++ks) load(ks);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      if (ks + kAhead < KSTEPS) load(ks + kAhead);
#pragma unroll
      for (int mb = 0; mb < MBW; ++mb)
        sacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_t, a[ks % (kAhead + 1)][mb]), qf[ks],
            ks == 0 ? (f32x16_t){} : sacc[mb], 0, 0, 0);
    }
    // scheduling pattern: the first kAhead + 1 k-steps of reads, then one
    // k-step of products and one of reads in turn, then the last products
    __builtin_amdgcn_sched_group_barrier(0x100, (kAhead + 1) * MBW, 0);
#pragma unroll
    for (int ks = 0; ks < KSTEPS - kAhead - 1; ++ks) {
      __builtin_amdgcn_sched_group_barrier(0x008, MBW, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, MBW, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, (kAhead + 1) * MBW, 0);
  };
  // P = exp2(S * scale_log2 - mu) rounded to bf16 (the P^T operand), row sum
  auto softmax_p = [&](const f32x16_t (&sacc)[MBW], float mu, bf16x8_t (&pb)[2 * MBW]) -> float {
    float part = 0.f;
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = __builtin_amdgcn_exp2f(fmaf(sacc[mb][r], c2, -mu));
        part += e;
        pb[mb * 2 + (r >> 3)][r & 7] = (__bf16)e;
      }
    }
    return part;
  };
  // O^T += V^T P^T.  The A operand (V^T: 32 dims x 16 keys per lane block)
  // comes from the [key][D] page with ds_read_b64_tr_b16: in each group of 16
  // lanes, lane 4k+q reads 4 dims (4q..4q+3 of the group's 16) of key row k,
  // and the transposed result gives lane i those 4 keys of dim i.  Keys of a
  // lane's operand follow the S^T accumulator order: 16ks + 8r + 4hf + 0..3
  // for the two reads r.  Read offsets per (r, dim block); ks adds 16 rows.
  int vtr[2][DBLK];
  {
    const int tr_row = 4 * hf + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int row_r = 8 * r + tr_row;
#pragma unroll
      for (int md = 0; md < DBLK; ++md) {
        const int colx = md * 32 + tr_col;
        vtr[r][md] = PageLayout<D>::offset(row_r, colx >> 3) + ((colx & 7) << 1);
      }
    }
  }
  auto pv = [&](int stage, const bf16x8_t (&pb)[2 * MBW]) {
#pragma unroll
    for (int ks = 0; ks < 2 * MBW; ++ks) {
      const unsigned char* vb = vbuf_of(stage, kPair ? ph : ks >> 2);
#pragma unroll
      for (int md = 0; md < DBLK; ++md) {
        u32x4_t a;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const v4i16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4i16_t*)(vb + vtr[r][md] +
                                                            (ks & 3) * (32 * D)));
          const u32x2_t w = __builtin_bit_cast(u32x2_t, v);
          a[2 * r] = w[0];
          a[2 * r + 1] = w[1];
        }
        o[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), pb[ks],
                                                        o[md], 0, 0, 0);
      }
    }
  };
  // Key rows past the end of the sequence in its last block may hold anything
  // (P is 0 there, but 0 * NaN is not; a page past the end was not copied):
  // zero them in the V pages before P V.
  auto zero_v_tail = [&](int stage, int valid_keys) {
    constexpr int kRowChunks = D / 8;
#pragma unroll
    for (int s = 0; s < PPB; ++s) {
      const int valid = min(max(valid_keys - s * kPage, 0), kPage);
      unsigned char* vb = vbuf_of(stage, s);
      for (int f = valid * kRowChunks + tid; f < kPage * kRowChunks; f += NT)
        *reinterpret_cast<u32x4_t*>(vb + f * 16) = (u32x4_t){0u, 0u, 0u, 0u};
    }
  };
  // causal / end-of-sequence mask (diagonal and tail blocks only), then the
  // row's block max in log2 units
  auto mask_max = [&](int block, f32x16_t (&sacc)[MBW]) -> float {
    // keys of this wavefront's share of the block
    const int key0 = block * KVB + (kPair ? ph * kPage : 0);
    constexpr int KW = kPair ? kPage : KVB;
    if ((key0 + KW - 1 > wave_q0) || (key0 + KW > L)) {
      const int lim = min(qpos, L - 1) - key0 - 4 * hf;
#pragma unroll
      for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int koff = mb * 32 + 8 * (r >> 2) + (r & 3);
          sacc[mb][r] = koff > lim ? kNegInf : sacc[mb][r];
        }
    }
    float mx = kNegInf;
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[mb][r]);
    return pair_max(mx) * c2;
  };
  // returns this wavefront's own vote (uniform): without it the tile-wide AND
  // is false whatever the other wavefronts voted
  auto vote = [&](float bmx, int vb) -> bool {
    if (!skip_on) return false;
    const bool pred = !row_valid || (bmx < m_true - tau_l2);
    const bool wave_all = __all(pred);
    if (lane == 0) sVote[vb][wave] = wave_all ? 1 : 0;
    return wave_all;
  };

  // Block loop, one workgroup barrier per visited logical block.  Step t
  // (LDS stage t % NS): S(t) from the K pages already in LDS, mask, block max
  // and the tile vote; wait for this wavefront's copies of V(t) and K(t+1)
  // (issued NS - 1 steps earlier; the later ones stay in flight), barrier;
  // read the vote; start the copies of K(t+NS) and V(t+NS-1) into the stages
  // whose last readers have passed the barrier (HBM -> LDS); then the softmax
  // and P V of block t unless the head's tile skips it.
  // With four stages every step issues the same copies (past the last slot
  // they repeat the last slot's pages into stages no later step reads), so
  // that the count of copies in flight is the same on every path and the
  // compiler can tell which ones a wait covers.
  if (cnt > 0) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int ts = NS == 4 ? min(s, cnt - 1) : s;
      if ((NS == 4 || s < cnt) && selected(ts)) copy_k(ts, slot_block(ts), s);
    }
#pragma unroll
    for (int s = 0; s + 1 < NS; ++s) {
      const int ts = NS == 4 ? min(s, cnt - 1) : s;
      if ((NS == 4 || s < cnt) && selected(ts)) copy_v(ts, slot_block(ts), s);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  // The ring entries a step needs (its block, and the pages of the copies it
  // starts) are read during the step before, after its barrier, and moved
  // to scalar registers at its end, so that a step's first LDS reads are its
  // K operands and no LDS load is pending across the loop's back edge.  The
  // ring holds those slots by then and no refill writes their half (a refill
  // targets the chunk 64 slots ahead).
  struct NextRefs {
    int block;      // slot t's logical block (ordered walk)
    SlotRef k, v;   // the slots whose K and V pages step t copies
  };
  auto read_next = [&](int t) -> NextRefs {
    NextRefs r;
    r.block = kOrdered ? sSlotB[(t >> 6) & 1][t & 63] : t;
    r.k = slot_ref(NS == 4 ? min(t + NS, cnt - 1) : t + NS);
    r.v = slot_ref(NS == 4 ? min(t + NS - 1, cnt - 1) : t + NS - 1);
    return r;
  };
  auto uniform_refs = [&](const NextRefs& r) -> NextRefs {
    NextRefs u;
    u.block = __builtin_amdgcn_readfirstlane(r.block);
#pragma unroll
    for (int s = 0; s < PPB; ++s) {
      u.k.page[s] = __builtin_amdgcn_readfirstlane(r.k.page[s]);
      u.v.page[s] = __builtin_amdgcn_readfirstlane(r.v.page[s]);
    }
    u.k.block = __builtin_amdgcn_readfirstlane(r.k.block);
    u.v.block = __builtin_amdgcn_readfirstlane(r.v.block);
    return u;
  };
  NextRefs nx = uniform_refs(read_next(0));
  // One step per slot; the slot's LDS stage (t % NS) is a compile-time
  // constant, so every LDS operand address is a fixed per-lane offset plus an
  // immediate.
  auto step = [&](const int t, auto stage_c) {
    constexpr int st = decltype(stage_c)::value;     // t % NS
    constexpr int vb = st & 1;                       // vote buffer, t & 1
    constexpr int st_prev = (st + NS - 1) % NS;      // stage of slot t - 1 and t + NS - 1
    const int j_cur = kOrdered ? nx.block : t;
    const int key0 = j_cur * KVB;
    const bool sel = selected(t);
    // the slots whose copies this step starts
    const int tk = NS == 4 ? min(t + NS, cnt - 1) : t + NS;
    const int tv = NS == 4 ? min(t + NS - 1, cnt - 1) : t + NS - 1;
    const SlotRef ref_k = nx.k;
    const SlotRef ref_v = nx.v;
    // some key of the block is visible to some valid row of this wave
    const bool active = sel && wave_has_rows && key0 <= wave_last;
    f32x16_t sacc[MBW];
    float bm = kNegInf;
    // The logits do not wait for the slot's block id: on the ordered and
    // dense walks they are formed for every slot (a block outside this
    // wave's rows is masked to -inf, the value side stays gated); only the
    // logical walk leaves unselected blocks out.
    if (!kLogical || active) {
      qk(st, sacc);
      bm = mask_max(j_cur, sacc);
    }
    // (two-page blocks: this wavefront's page only; the block is skipped
    // when both pages are, since its max is below the threshold exactly when
    // both pages' maxima are)
    const bool own_vote = vote(bm, vb);
    if constexpr (kPair) {
      if (hf == 0) sBm[vb][ph][wv * 32 + col] = bm;
    }
    // V(t) and K(t+1) were issued NS - 1 steps ago; the copies of the NS - 2
    // steps since then stay in flight
    wait_vm_c<(NS - 2) * 2 * K_PER * PPB>();
    lds_barrier();
    // the block's row max over both pages
    if constexpr (kPair) bm = fmaxf(bm, sBm[vb][1 - ph][wv * 32 + col]);

    bool skip = false;
    if (own_vote) {
      int all = 1;
      constexpr int NV = kPair ? NWT : NW;   // wavefronts that vote on this block
#pragma unroll
      for (int w = 0; w < NV; ++w) all &= sVote[vb][(kPair ? 0 : hs * NW) + w];
      skip = __builtin_amdgcn_readfirstlane(all) != 0;   // uniform over the head
    }
    if (kOrdered) {
      nskip += skip ? 1 : 0;
      if (p.skip_record != nullptr) {
        // every lane keeps the (uniform) word; the head writer stores it
        rec_word |= (skip ? 1u : 0u) << (t & 31);
        if ((t & 31) == 31 || t + 1 == cnt) {
          if (head_writer) sRec[hs][t >> 5] = rec_word;
          rec_word = 0;
        }
      }
    }

    // ---- prefetch: K(t+NS) and V(t+NS-1) straight into LDS, and the slot
    // chunk after the one that holds slot t+1.  The refill of that chunk
    // overwrites the ring half holding slot t's own entries (chunks c+1 and
    // c-1 share a half), so it comes after the last read of slot t's pages:
    // the on-demand V fetch below.
    if constexpr (NS == 4) {
      advance_chunks(t + 1);
      copy_ref(p.k_pool, ref_k, st, true);
      copy_ref(p.v_pool, ref_v, st_prev, false);
    } else {
      // A skipped block needs no V page.  Skips come in runs (once the row
      // maxima are found, most later blocks fall below them), so V(t+1) is
      // prefetched only after a computed block; a computed block whose V was
      // not prefetched fetches it here, before the other copies, and waits.
      if (sel && !skip && !v_have) {   // uniform over the workgroup
        copy_v(t, j_cur, st);
        wait_vm_c<0>();
        lds_barrier();                 // every wave has read slot t's pages
      }
      advance_chunks(t + 1);
      if (tk < cnt && selected(tk)) copy_ref(p.k_pool, ref_k, st, true);
      v_have = false;
      if (tv < cnt && selected(tv) && !skip) {
        copy_ref(p.v_pool, ref_v, st_prev, false);
        v_have = true;
      }
    }

    if (sel && key0 + KVB > L) {   // uniform: the sequence's last block
      zero_v_tail(st, L - key0);
      __syncthreads();
    }
    const NextRefs nx_raw = read_next(t + 1);
    if (active && !skip) {
      // ---- online softmax (log2 domain) with lazy rescaling
      const float mn = fmaxf(m_true, bm);
      m_true = mn;
      const bool need = mn > m_ref + kRescale;
      if (__any(need)) {
        const float new_ref = need ? mn : m_ref;
        const float alpha = (m_ref == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m_ref - new_ref);
        m_ref = new_ref;
        lsum *= alpha;
#pragma unroll
        for (int md = 0; md < DBLK; ++md) o[md] *= alpha;
      }
      const float mu = (m_ref == kNegInf) ? 0.f : m_ref;
      bf16x8_t pb[2 * MBW];
      lsum += softmax_p(sacc, mu, pb);
      pv(st, pb);
    }
    nx = uniform_refs(nx_raw);
  };
  // Whole groups of NS steps in the loop, the rest after it: every path
  // around the loop issues the same copies.
  int t0 = 0;
  for (; t0 + NS <= cnt; t0 += NS) {
    step(t0, std::integral_constant<int, 0>{});
    step(t0 + 1, std::integral_constant<int, 1>{});
    if constexpr (NS == 4) {
      step(t0 + 2, std::integral_constant<int, 2>{});
      step(t0 + 3, std::integral_constant<int, 3>{});
    }
  }
  if (t0 < cnt) step(t0, std::integral_constant<int, 0>{});
  if constexpr (NS == 4) {
    if (t0 + 1 < cnt) step(t0 + 1, std::integral_constant<int, 1>{});
    if (t0 + 2 < cnt) step(t0 + 2, std::integral_constant<int, 2>{});
  }

  // ---- two-page blocks: page half 1 adds its partial O and row sums into
  // half 0's through LDS (the page buffers are free after the last step;
  // both halves hold the same running max and reference)
  if constexpr (kPair) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();   // every wavefront is past its last read of the pages
    float* xo = reinterpret_cast<float*>(kraw(wv));
    float* xl = reinterpret_cast<float*>(sV0) + wv * 64;
    if (ph == 1) {
#pragma unroll
      for (int md = 0; md < DBLK; ++md)
#pragma unroll
        for (int r = 0; r < 16; ++r) xo[(md * 16 + r) * 64 + lane] = o[md][r];
      xl[lane] = lsum;
    }
    __syncthreads();
    if (ph == 0) {
#pragma unroll
      for (int md = 0; md < DBLK; ++md)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[md][r] += xo[(md * 16 + r) * 64 + lane];
      lsum += xl[lane];
    }
  }
  // ---- epilogue: out = O / l, lse = m + ln l
  const float ltot = pair_sum(lsum);
  if (row_valid && ph == 0) {
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    uint16_t* dst = p.out + ((int64_t)(q0 + qpos) * p.hq + h) * D;
#pragma unroll
    for (int md = 0; md < DBLK; ++md) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d = md * 32 + 8 * rq + 4 * hf;
        __bf16 v4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(o[md][4 * rq + e] * inv);
        u32x2_t w;
        w[0] = (uint32_t)__builtin_bit_cast(uint16_t, v4[0]) |
               ((uint32_t)__builtin_bit_cast(uint16_t, v4[1]) << 16);
        w[1] = (uint32_t)__builtin_bit_cast(uint16_t, v4[2]) |
               ((uint32_t)__builtin_bit_cast(uint16_t, v4[3]) << 16);
        *reinterpret_cast<u32x2_t*>(dst + d) = w;
      }
    }
    if (p.lse != nullptr && hf == 0) {
      p.lse[(int64_t)h * p.total_q + q0 + qpos] =
          ltot > 0.f ? (m_ref + __log2f(ltot)) * kLn2 : kNegInf;
    }
  }
  if (kOrdered && p.row_stats != nullptr && head_writer) {
    p.row_stats[2 * row] = cnt;
    p.row_stats[2 * row + 1] = nskip;
  }
  if (kOrdered && p.skip_record != nullptr) {
    __syncthreads();   // every head writer's last record word is in LDS
    uint8_t* rec = p.skip_record + row * p.capacity;
    if (ph == 0)
      for (int t = tid_h; t < cnt; t += NTH)
        rec[t] = (uint8_t)((sRec[hs][t >> 5] >> (t & 31)) & 1u);
  }
}

// Dense walk with two query heads of a KV group per workgroup, the two heads
// in opposite phases.  Wavefront w of head 0 and wavefront w of head 1 share
// a SIMD (the waves of a workgroup go round-robin over the four SIMDs), so
// when both heads run the same part of the page step at once, the matrix
// core idles while both do the softmax on the VALU and the VALU idles while
// both issue products.  Here each head's step is split into a product phase
// M(t) = P V(t-1) then S(t) = K(t) Q^T (32 MFMAs per wavefront) and a vector
// phase V(t) = mask, block max, rescale, P(t) = exp2(S(t) - mu) and its row
// sum, and the heads take turns:
//
//     phase 2t     head 0: M(t)      head 1: V(t-1)
//     phase 2t+1   head 0: V(t)      head 1: M(t)
//
// with one workgroup barrier per phase; the head in its product phase runs at
// a raised wave priority, and the page copies are issued at the start of the
// vector phases, the K pages by head 1 and the V pages by head 0.  Each head still visits every causal block in ascending
// order and applies the same arithmetic in the same order as the one-phase
// step, so its output is the same bit for bit.  K(t) is read in phases 2t and
// 2t+1 and V(t-1) in the same two, so after phase 2t+1 their LDS stages take
// K(t+4) and V(t+3); the copies run three blocks ahead (four LDS stages per
// operand, 128 KB, one workgroup per CU).
template <int D>
__global__ __launch_bounds__(512, 1) void attn_dense_pp_kernel(const AttnParams p) {
  constexpr int NW = 4;                      // wavefronts per head, 32 query rows each
  constexpr int NT = 2 * NW * 64;            // two heads
  constexpr int BQ = NW * 32;                // query rows per tile
  constexpr int NS = 4;                      // LDS stages per operand
  constexpr int KCH = D / 8;                 // 16-byte chunks per key row
  constexpr int K_TOTAL = kPage * KCH;       // 16-byte chunks per page
  static_assert(K_TOTAL % NT == 0, "page copy must split evenly over the workgroup");
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;
  constexpr float kRescale = 8.f;
  constexpr int kBytes = PageLayout<D>::kBytes;

  __shared__ __attribute__((aligned(16))) unsigned char sK0[kBytes];
  __shared__ __attribute__((aligned(16))) unsigned char sK1[kBytes];
  __shared__ __attribute__((aligned(16))) unsigned char sK2[kBytes];
  __shared__ __attribute__((aligned(16))) unsigned char sK3[kBytes];
  __shared__ __attribute__((aligned(16))) unsigned char sV0[kBytes];
  __shared__ __attribute__((aligned(16))) unsigned char sV1[kBytes];
  __shared__ __attribute__((aligned(16))) unsigned char sV2[kBytes];
  __shared__ __attribute__((aligned(16))) unsigned char sV3[kBytes];
  __shared__ int sSlotP[2][64];   // [ring chunk][slot]: page of causal block
  auto kbuf = [&](int x) -> unsigned char* {
    return x == 0 ? sK0 : x == 1 ? sK1 : x == 2 ? sK2 : sK3;
  };
  auto vbuf = [&](int x) -> unsigned char* {
    return x == 0 ? sV0 : x == 1 ? sV1 : x == 2 ? sV2 : sV3;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave / NW;                 // head of the workgroup (0 or 1)
  const int wv = wave - grp * NW;
  const int hf = lane >> 5;
  const int col = lane & 31;

  int b, hu, i;
  decode_tile(p, blockIdx.x, p.hq / 2, b, hu, i);
  const int h = hu * 2 + grp;
  const int g = (hu * 2) / (p.hq / p.hkv);
  const int q0 = p.cu_seqlens[b];
  const int L = p.cu_seqlens[b + 1] - q0;
  const int tile_q0 = i * BQ;
  if (tile_q0 >= L) return;
  const int tile_last = min(tile_q0 + BQ, L) - 1;
  const int cnt = tile_last / kPage + 1;
  const int32_t* __restrict__ pt = p.page_table + (int64_t)b * p.max_pages;

  const int wave_q0 = tile_q0 + wv * 32;
  const int wave_last = min(wave_q0 + 31, L - 1);
  const int qpos = wave_q0 + col;
  const bool row_valid = qpos < L;
  const bool wave_has_rows = wave_q0 < L;

  bf16x8_t qf[KSTEPS];
  {
    const uint16_t* qp = p.q + ((int64_t)(q0 + qpos) * p.hq + h) * D + hf * 8;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (row_valid) v = *reinterpret_cast<const u32x4_t*>(qp + ks * 16);
      qf[ks] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // Page ids of the causal blocks from a two-chunk ring of 64 entries in LDS.
  // Chunk c (slots 64c..) is copied into half c & 1 by the first wavefront
  // of head 1 at the start of block 64c - 6, before that block's K copies.
  // Every wait for copies lets only the page copies of the two latest blocks
  // stay in flight, so the chunk has landed by the first barrier of block
  // 64c - 4 at the latest; slot 64c is first read in the second phase of that
  // block.  The half's previous chunk (c - 2) was last read in block 64c - 68.
  if (wave == 0) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int x = c * 64 + lane;
      sSlotP[c][lane] = x < cnt ? pt[x] : 0;
    }
  }
  __syncthreads();
  auto slot_page = [&](int t) -> int { return sSlotP[(t >> 6) & 1][t & 63]; };

  const int64_t head_stride = (int64_t)kPage * D;
  const int64_t page_stride = (int64_t)p.hkv * head_stride;
  // Each head copies one operand's pages (K_PER copy instructions per page
  // and wavefront), head 1 the K pages and head 0 the V pages, each in the
  // phase where that head runs its vector work, so the head issuing products
  // never waits for room in the vector-memory queue.
  constexpr int NC = NW * 64;                // copying threads of a head
  constexpr int K_PER = K_TOTAL / NC;
  const int tidc = tid - grp * NC;
  uint32_t coff[K_PER];
#pragma unroll
  for (int e = 0; e < K_PER; ++e) {
    const int f = e * NC + tidc;
    const int r = f / KCH;
    const int c = (f % KCH) ^ PageLayout<D>::swz(r);
    coff[e] = (uint32_t)(r * D + c * 8) * 2u;
  }
  constexpr int kSliceBytes = kPage * D * 2;
  auto copy_page = [&](const uint16_t* pool, int page, unsigned char* dst) __attribute__((always_inline)) {
    const uint16_t* base = pool + (int64_t)page * page_stride + (int64_t)g * head_stride;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(base), (short)0, kSliceBytes, kBufferWord3);
#pragma unroll
    for (int e = 0; e < K_PER; ++e) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(dst + (e * NC + wv * 64) * 16), 16,
          (int)coff[e], 0, 0, 0);
    }
  };

  f32x16_t o[DBLK];
#pragma unroll
  for (int md = 0; md < DBLK; ++md) o[md] = (f32x16_t){};
  float m_true = kNegInf;
  float m_ref = kNegInf;
  float lsum = 0.f;
  const float c2 = p.scale_log2;

  // S^T(block) = K Q^T for this wave's 32 queries, K operand reads two
  // k-steps ahead of the products
  auto qk = [&](const unsigned char* kb, f32x16_t (&sacc)[2]) __attribute__((always_inline)) {
    constexpr int kAhead = 2;
    u32x4_t a[kAhead + 1][2];
    auto load = [&](int ks) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        a[ks % (kAhead + 1)][mb] = *reinterpret_cast<const u32x4_t*>(
            kb + PageLayout<D>::offset(mb * 32 + col, 2 * ks + hf));
    };
#pragma unroll
    for (int ks = 0; ks < kAhead; ++ks) load(ks);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      if (ks + kAhead < KSTEPS) load(ks + kAhead);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        sacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_t, a[ks % (kAhead + 1)][mb]), qf[ks],
            ks == 0 ? (f32x16_t){} : sacc[mb], 0, 0, 0);
    }
    // the first kAhead + 1 k-steps of reads, then one k-step of products
    // and one of reads in turn, then the last products
    __builtin_amdgcn_sched_group_barrier(0x100, (kAhead + 1) * 2, 0);
#pragma unroll
    for (int ks = 0; ks < KSTEPS - kAhead - 1; ++ks) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, (kAhead + 1) * 2, 0);
  };
  int vtr[2][DBLK];
  {
    const int tr_row = 4 * hf + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int row_r = 8 * r + tr_row;
#pragma unroll
      for (int md = 0; md < DBLK; ++md) {
        const int colx = md * 32 + tr_col;
        vtr[r][md] = PageLayout<D>::offset(row_r, colx >> 3) + ((colx & 7) << 1);
      }
    }
  }
  // O^T += V^T P^T (transposing LDS reads of the [key][D] page)
  // V^T operand of product k = 4 ks + md (md < DBLK) of P V
  auto pv_operand = [&](const unsigned char* vb, int k) __attribute__((always_inline)) -> u32x4_t {
    const int ks = k / DBLK, md = k % DBLK;
    u32x4_t a;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const v4i16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4i16_t*)(vb + vtr[r][md] + ks * (32 * D)));
      const u32x2_t w = __builtin_bit_cast(u32x2_t, v);
      a[2 * r] = w[0];
      a[2 * r + 1] = w[1];
    }
    return a;
  };
  auto pv = [&](const unsigned char* vb, const bf16x8_t (&pb)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 4 * DBLK; ++k) {
      const u32x4_t a = pv_operand(vb, k);
      o[k % DBLK] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                            pb[k / DBLK], o[k % DBLK], 0, 0, 0);
    }
    // operand reads three products ahead
    constexpr int kAhead = 3;
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAhead, 0);
#pragma unroll
    for (int k = 0; k < 4 * DBLK - kAhead; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
  };
  // the vector phase of block s: causal / end mask, block max, online-softmax
  // update with lazy rescaling, P(s) as the bf16 operand of P V and its row sum
  auto vphase = [&](int s, f32x16_t (&sacc)[2], bf16x8_t (&pb)[4]) __attribute__((always_inline)) {
    const int key0 = s * kPage;
    if ((key0 + kPage - 1 > wave_q0) || (key0 + kPage > L)) {
      const int lim = min(qpos, L - 1) - key0 - 4 * hf;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int koff = mb * 32 + 8 * (r >> 2) + (r & 3);
          sacc[mb][r] = koff > lim ? kNegInf : sacc[mb][r];
        }
    }
    float mx = kNegInf;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[mb][r]);
    const float bm = pair_max(mx) * c2;
    const float mn = fmaxf(m_true, bm);
    m_true = mn;
    const bool need = mn > m_ref + kRescale;
    if (__any(need)) {
      const float new_ref = need ? mn : m_ref;
      const float alpha = (m_ref == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m_ref - new_ref);
      m_ref = new_ref;
      lsum *= alpha;
#pragma unroll
      for (int md = 0; md < DBLK; ++md) o[md] *= alpha;
    }
    const float mu = (m_ref == kNegInf) ? 0.f : m_ref;
    float part = 0.f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = __builtin_amdgcn_exp2f(fmaf(sacc[mb][r], c2, -mu));
        part += e;
        pb[mb * 2 + (r >> 3)][r & 7] = (__bf16)e;
      }
    }
    lsum += part;
  };
  // some key of block s is visible to some valid row of this wave
  auto active = [&](int s) -> bool { return wave_has_rows && s * kPage <= wave_last; };

  // prologue: K(0..2) and V(0..1); past the last block the copies repeat the
  // last block's page into stages no step reads
  if (grp == 1) {
#pragma unroll
    for (int s = 0; s < NS - 1; ++s) copy_page(p.k_pool, pt[min(s, cnt - 1)], kbuf(s));
#pragma unroll
    for (int s = 0; s < NS - 2; ++s) copy_page(p.v_pool, pt[min(s, cnt - 1)], vbuf(s));
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  f32x16_t sacc[2];
  bf16x8_t pb[4];
  // pages of the copies the next block starts (uniform)
  int nk = __builtin_amdgcn_readfirstlane(slot_page(min(NS - 1, cnt - 1)));
  int nv = __builtin_amdgcn_readfirstlane(slot_page(min(NS - 2, cnt - 1)));

  // One block: its two phases; stage of K(t) is t % NS, of V(t - 1) is
  // (t - 1) % NS.  Each head runs its own copy of the loop (kB: head 1), so
  // that the register allocation of each is its own; both pass the same
  // barriers in the same order.
  auto block = [&](const int t, auto stage_c, auto head_c) __attribute__((always_inline)) {
    constexpr int sk = decltype(stage_c)::value;
    constexpr int sv = (sk + NS - 1) % NS;
    constexpr bool kB = decltype(head_c)::value;
    // ---- phase 2t.  K(t) (head 1's copy) and V(t - 1) (head 0's) were
    // copied three blocks ago; each head's copies of the two blocks since
    // stay in flight.
    wait_vm_c<2 * K_PER>();
    lds_barrier();
    if (kB && wv == 0 && ((t + 6) & 63) == 0 && t + 6 >= 128 && t + 6 < cnt) {
      const int c = (t + 6) >> 6;
      const int x = min(c * 64 + lane, cnt - 1);
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(pt + x),
                                       (__attribute__((address_space(3))) void*)&sSlotP[c & 1][0],
                                       4, 0, 0);
    }
    // K(t + 3) into the stage of K(t - 1)
    if constexpr (kB) copy_page(p.k_pool, nk, kbuf((sk + NS - 1) % NS));
    const bool pv_on = t > 0 && active(t - 1);
    const bool qk_on = active(t);
    // the head issuing products takes issue priority over the other
    if constexpr (!kB) {
      __builtin_amdgcn_s_setprio(1);
      if (pv_on) pv(vbuf(sv), pb);
      if (qk_on) qk(kbuf(sk), sacc);
      __builtin_amdgcn_s_setprio(0);
    } else {
      if (pv_on) vphase(t - 1, sacc, pb);
    }
    // ---- phase 2t + 1
    lds_barrier();
    const int rk = slot_page(min(t + NS, cnt - 1));
    const int rv = slot_page(min(t + NS - 1, cnt - 1));
    if constexpr (!kB) {
      // V(t + 2) into the stage of V(t - 2), read last in phase 2t - 1
      copy_page(p.v_pool, nv, vbuf((sk + 2) % NS));
      if (qk_on) vphase(t, sacc, pb);
    } else {
      __builtin_amdgcn_s_setprio(1);
      if (pv_on) pv(vbuf(sv), pb);
      if (qk_on) qk(kbuf(sk), sacc);
      __builtin_amdgcn_s_setprio(0);
    }
    nk = __builtin_amdgcn_readfirstlane(rk);
    nv = __builtin_amdgcn_readfirstlane(rv);
  };
  auto run = [&](auto head_c) __attribute__((always_inline)) {
    constexpr bool kB = decltype(head_c)::value;
    int t0 = 0;
    for (; t0 + NS <= cnt; t0 += NS) {
      block(t0, std::integral_constant<int, 0>{}, head_c);
      block(t0 + 1, std::integral_constant<int, 1>{}, head_c);
      block(t0 + 2, std::integral_constant<int, 2>{}, head_c);
      block(t0 + 3, std::integral_constant<int, 3>{}, head_c);
    }
    if (t0 < cnt) block(t0, std::integral_constant<int, 0>{}, head_c);
    if (t0 + 1 < cnt) block(t0 + 1, std::integral_constant<int, 1>{}, head_c);
    if (t0 + 2 < cnt) block(t0 + 2, std::integral_constant<int, 2>{}, head_c);

    // ---- drain: P V of the last block, after its V page's tail past the
    // end of the sequence (P is 0 there, 0 * NaN is not) is zeroed
    const int last = cnt - 1;
    unsigned char* vl = vbuf(last & (NS - 1));
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();
    if (last * kPage + kPage > L) {
      const int valid = L - last * kPage;
      for (int f = valid * KCH + tid; f < kPage * KCH; f += NT)
        *reinterpret_cast<u32x4_t*>(vl + f * 16) = (u32x4_t){0u, 0u, 0u, 0u};
      lds_barrier();
    }
    const bool last_on = active(last);
    if constexpr (!kB) {
      if (last_on) pv(vl, pb);
      lds_barrier();
    } else {
      if (last_on) vphase(last, sacc, pb);
      lds_barrier();
      if (last_on) pv(vl, pb);
    }
  };
  if (grp == 0)
    run(std::false_type{});
  else
    run(std::true_type{});

  // ---- epilogue: out = O / l, lse = m + ln l
  const float ltot = pair_sum(lsum);
  if (row_valid) {
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    uint16_t* dst = p.out + ((int64_t)(q0 + qpos) * p.hq + h) * D;
#pragma unroll
    for (int md = 0; md < DBLK; ++md) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d = md * 32 + 8 * rq + 4 * hf;
        __bf16 v4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(o[md][4 * rq + e] * inv);
        u32x2_t w;
        w[0] = (uint32_t)__builtin_bit_cast(uint16_t, v4[0]) |
               ((uint32_t)__builtin_bit_cast(uint16_t, v4[1]) << 16);
        w[1] = (uint32_t)__builtin_bit_cast(uint16_t, v4[2]) |
               ((uint32_t)__builtin_bit_cast(uint16_t, v4[3]) << 16);
        *reinterpret_cast<u32x2_t*>(dst + d) = w;
      }
    }
    if (p.lse != nullptr && hf == 0) {
      p.lse[(int64_t)h * p.total_q + q0 + qpos] =
          ltot > 0.f ? (m_ref + __log2f(ltot)) * kLn2 : kNegInf;
    }
  }
}

template <int D, int NW, int kMode, int PPB, int HP, int NS>
hipError_t launch_one(const AttnParams& p, hipStream_t stream) {
  const int64_t n_groups = p.group_count > 0 ? p.group_count : (int64_t)p.batch * p.hkv;
  const int64_t grid = n_groups * (p.hq / p.hkv / HP) * p.nqb;
  if (grid <= 0) return hipSuccess;
  // two-page blocks: a pair of wavefronts per 32 query rows
  hipLaunchKernelGGL((attn_fwd_kernel<D, NW, kMode, PPB, HP, NS>), dim3((unsigned)grid),
                     dim3(NW * (PPB == 2 ? 2 : HP) * 64), 0, stream, p);
  return hipGetLastError();
}

template <int D, int NW>
hipError_t launch_mode(const AttnParams& p, AttnMode mode, int ppb, hipStream_t stream) {
  if (ppb == 2) {
    if (mode == kModeOrdered) return launch_one<D, NW, kModeOrdered, 2, 1, 2>(p, stream);
    return hipErrorInvalidValue;
  }
  if (mode == kModeOrdered) return launch_one<D, NW, kModeOrdered, 1, 1, 2>(p, stream);
  if (mode == kModeLogical) return launch_one<D, NW, kModeLogical, 1, 1, 2>(p, stream);
  return launch_one<D, NW, kModeDense, 1, 1, 2>(p, stream);
}

// Two query heads per workgroup for the dense walk (every head of a KV group
// visits the same pages), four LDS stages.
hipError_t launch_dense_pairs(const AttnParams& p, hipStream_t stream) {
#if COSA_DENSE_PP
  const int64_t n_groups = p.group_count > 0 ? p.group_count : (int64_t)p.batch * p.hkv;
  const int64_t grid = n_groups * (p.hq / p.hkv / 2) * p.nqb;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(attn_dense_pp_kernel<128>, dim3((unsigned)grid), dim3(512), 0, stream, p);
  return hipGetLastError();
#else
  return launch_one<128, 4, kModeDense, 1, 2, 4>(p, stream);
#endif
}

}  // namespace

hipError_t launch_attention(const AttnParams& p, int head_dim, int q_block, AttnMode mode,
                            hipStream_t stream) {
  // a range of groups is only defined in the group-major order
  if (p.group_count > 0 && p.order != kOrderGroupMajor && p.order != kOrderGroupXcd)
    return hipErrorInvalidValue;
  // The dense walk visits every causal key in ascending order whatever the
  // logical block size, so it walks one 64-key page per step.
  const int ppb = mode == kModeDense ? 1 : p.ppb;
  if (COSA_HEAD_PAIRS && mode == kModeDense && head_dim == 128 && q_block == 128 &&
      (p.hq / p.hkv) % 2 == 0)
    return launch_dense_pairs(p, stream);
  if (head_dim == 128 && q_block == 128) return launch_mode<128, 4>(p, mode, ppb, stream);
  if (head_dim == 128 && q_block == 64) return launch_mode<128, 2>(p, mode, ppb, stream);
  if (head_dim == 64 && q_block == 128) return launch_mode<64, 4>(p, mode, ppb, stream);
  if (head_dim == 64 && q_block == 64) return launch_mode<64, 2>(p, mode, ppb, stream);
  return hipErrorInvalidValue;
}

}  // namespace cosa
