// Internal declarations shared by the host API and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cosa {

constexpr int kPage = 64;          // tokens per KV page == logical key block
constexpr int kProxyRows = 16;     // query rows pooled into one proxy row
constexpr int kMaxCandidates = 2048;  // KAP: key blocks per tile handled in one pass

// x plus the value of lane ^ 32, in one VALU exchange of the two 32-lane
// halves (v_permlane32_swap returns the lane's own value and its partner's;
// the sum is the same in either order).
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroup -> (sequence, head, tile) orders of the attention kernel.  All
// of them launch tiles with more causal blocks first.
enum TileOrder : int32_t {
  kOrderLevel = 0,      // tile level major, every head of the batch per level
  kOrderXcdGroup = 1,   // every KV group pinned to one XCD (needs B*Hkv % 8 == 0)
  kOrderGroupMajor = 2, // one KV group after the other: its K/V stay cache-resident
  kOrderGroupXcd = 3    // group-major, the query heads of one (group, tile) on one XCD
                        // (needs the launched groups' tile count % 8 == 0)
                        // (needs B*Hkv*NQB % 8 == 0)
};

// Arguments of the attention kernel (dense and ordered-skipping modes).
struct AttnParams {
  const uint16_t* q;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  uint16_t* out;
  float* lse;
  const int32_t* cu_seqlens;
  const int32_t* page_table;
  const int32_t* ordered_blocks;  // OSK only
  const int32_t* ordered_pages;   // OSK only
  const int32_t* counts;          // OSK only
  uint8_t* skip_record;           // OSK only, nullable
  int32_t* row_stats;             // OSK only, nullable
  int32_t mask_heads;             // OSK: heads of the mask layout (Hq, or Hkv when shared)
  int32_t ppb;                    // pages per logical key block (1 or 2)
  const uint32_t* block_mask;     // logical-skip mode only: [rows][mask_words] bits
  int64_t mask_words;
  int64_t capacity;
  int64_t total_q;
  int32_t batch, hq, hkv, max_pages, nqb;
  int32_t xcd_groups;             // B*Hkv when it is a multiple of 8, else 0
  int32_t xcd_units;              // B*Hkv*NQB when it is a multiple of 8, else 0
  int32_t order;                  // tile order, one of TileOrder
  // (sequence, KV head) groups [group_begin, group_begin + group_count) only
  // (group_count 0: every group); needs a group-major order
  int32_t group_begin, group_count;
  float scale_log2;               // softmax_scale * log2(e)
  int32_t skip_mode;              // OSK: kSkipOff, kSkipTau or kSkipDelta
  float tau_log2;                 // kSkipTau: threshold * log2(e)
  float log2_delta;               // kSkipDelta: log2(Delta); tau = log2(L_b) - log2(Delta)
};

// Page-walk modes of the attention kernel.
enum AttnMode : int32_t {
  kModeDense = 0,    // every causal block, ascending
  kModeOrdered = 1,  // the blocks of the ordered mask, in its order (OSK)
  kModeLogical = 2   // every causal block, ascending, computing only those whose
                     // bit is set in a block bitmask (logical mask skipping)
};

// In-kernel skip modes of the ordered-skipping kernel.
enum SkipMode : int32_t {
  kSkipOff = 0,    // every visited block is computed
  kSkipTau = 1,    // one threshold for every sequence
  kSkipDelta = 2   // length-adaptive: threshold ln(L_b / Delta) per sequence
};

// Arguments of the two KAP kernels.
struct KapParams {
  const uint16_t* q;
  const uint16_t* k_pool;
  const int32_t* cu_seqlens;
  const int32_t* page_table;
  // workspace: pooled keys, bf16 hi and lo planes, each [B][Hkv] of
  // ceil(n_max / 32) candidate groups laid out as the score product reads
  // them: [group][D / 16][2][32 blocks][8]
  uint16_t* kbar;
  int32_t* ordered_blocks;
  int32_t* ordered_pages;
  int32_t* counts;
  int32_t* hrm_counts;            // nullable
  float* debug_w;                 // nullable [rows][n_max]
  uint8_t* debug_hrm;             // nullable [rows][n_max]
  int64_t capacity;
  int32_t batch, hq, hkv, max_pages, nqb, n_max;
  int32_t kv_block;               // tokens per logical key block (1 or 2 pages)
  int32_t ppb;                    // pages per logical block
  int32_t beta_ppm;
  float scale;
  // Top-p mass in fixed point (p * 2^48, rounded down); 0 = budget only,
  // all ones = p of 1 (keep every candidate the budget allows)
  uint64_t top_p_fx;
  // 0: one mask per query head; else the number of query heads per KV head,
  // one mask per KV head shared by them
  int32_t shared_heads;
  // (sequence, KV head) groups [group_begin, group_begin + group_count) only
  // (group_count 0: every group)
  int32_t group_begin, group_count;
};

// Parts of the proxy to launch.
enum KapStage : int32_t { kKapPool = 1, kKapSelect = 2, kKapAll = 3 };

hipError_t launch_attention(const AttnParams& p, int head_dim, int q_block, AttnMode mode,
                            hipStream_t stream);
hipError_t launch_kap(const KapParams& p, int head_dim, int q_block, hipStream_t stream,
                      KapStage stage = kKapAll);

}  // namespace cosa
