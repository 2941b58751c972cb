// Internal declarations shared by the kernels and the C-ABI entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kPageSize = 16;      // tokens per page (S)
constexpr int kWaves = 4;          // waves per attention workgroup (independent work items but in prefill)
constexpr int kMaxGroup = 16;      // query heads per KV head held in one MFMA tile
constexpr int kMaxQLen = 8;        // query tokens per sequence in one multi-query call
constexpr int kMaxCols = 64;       // query columns (heads x tokens) per unit: 4 MFMA tiles
#ifndef PA_SHARED_PREFILL
#define PA_SHARED_PREFILL 1        // prefill: 32-column waves that share each page through LDS
#endif
// Query columns per wave of a prefill chunk (units of more than kMaxCols
// columns): 32 for the page-sharing kernel, else 64.
constexpr int kPrefillCols = PA_SHARED_PREFILL ? 32 : kMaxCols;
constexpr int kMassRun = 128;      // pages per wave of the eviction score pass (LDS rows)

// Arguments of the attention (partial) kernel.
struct AttnArgs {
  const uint8_t* k_pages;
  const uint8_t* v_pages;
  const float* k_scale;      // FP8 only
  const float* v_scale;      // FP8 only
  const int32_t* block_table;
  const int32_t* lens;
  const uint32_t* flags;     // nullptr: nothing flagged; SEQ: per sequence
  // HEAD layout with the check on: one validation word per unit (the
  // sequence is flagged when any of its Hkv words is), and the sequence
  // words are written out by the last kernel of the decode (flags_out).
  const uint32_t* unit_flags;
  uint32_t* flags_out;
  int write_flags;           // this kernel writes flags_out[b] = OR of the unit words
  const uint16_t* q;         // [B][q_len][Hq][D]
  uint16_t* out;             // [B][q_len][Hq][D]; written directly when num_parts == 1
  float* part_o;             // [B][q_len][Hq][Pn][D] unnormalised outputs
  float* part_ml;            // [B][q_len][Hq][Pn][2] running max (log2 domain) and sum
  int batch, num_q_heads, num_kv_heads, group, table_width, num_pages;
  int q_len;                 // query tokens per sequence (1: decode; > 1: causal drafts)
  int col_blocks;            // blocks of kPrefillCols query columns per unit (prefill chunks); else 1
  float* row_ml;             // scored decode: [B][Hq][2] final max (log2) and sum per row
  float* scores;             // eviction score pass: [P][Hkv (SEQ) or 1 (HEAD)][S] page scores
  int chunk_pages, num_parts;
  int parts_per_wave;        // consecutive partitions of one unit a wave streams through
  int xcd_order;             // workgroup order that keeps a page's heads on one XCD
  float score_scale_log2;    // softmax_scale * log2(e)
  // Length-balanced split (automatic partitions; nullptr: fixed partitions of
  // chunk_pages).  Written by plan_block: plan[0] the chunk in pages,
  // plan[1] the number of pairs, plan[2 + g] the first pair of group g
  // (groups + 1 entries); plan_group[pair] the group of each pair.  A group
  // is a sequence (SEQ: its Hkv heads share the pair) or a unit (HEAD); a
  // pair is one partition of a group, and its partials sit in slots
  // pair * heads_per_group + head.
  const int32_t* plan;
  const int32_t* plan_group;
  // plan_rec[4 pair ..]: (group, partition within it, chunk, the group's
  // length) of each pair slot < max_pairs, group -1 past the last pair: what
  // an attention wave needs, in one load instead of three dependent ones.
  const int32_t* plan_rec;
  int max_pairs;
};

// Arguments of the length-balanced split planner.
struct PlanArgs {
  const int32_t* lens;       // one length per group
  int32_t* plan;             // as AttnArgs::plan
  int32_t* plan_group;
  int32_t* plan_rec;         // as AttnArgs::plan_rec; may be null
  int num_groups, heads_per_group, table_width, max_pairs;
  int target_waves, min_chunk, max_chunk;
};

struct ValidateArgs {
  const int32_t* block_table;
  const int32_t* lens;
  const uint32_t* expected_tags;  // nullptr: range and length checks only
  const uint32_t* page_tags;
  uint32_t* flags;                // per sequence, or per unit with per_unit
  int batch, num_kv_heads, table_width, num_pages;
  bool head_layout;
  bool per_unit;                  // HEAD: one workgroup and one word per unit
  int rows;                       // workgroups: batch, or batch * num_kv_heads with per_unit
};

struct AppendArgs {
  uint8_t* k_pages;
  uint8_t* v_pages;
  float* k_scale;
  float* v_scale;
  const int32_t* block_table;
  const int32_t* lens_old;
  const int32_t* n_new;
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint32_t* flags;
  // With expected_tags (the table's shape) a page is written only while its
  // tag is the one the request expects: a stale entry may name a page that
  // now belongs to another request.
  const uint32_t* expected_tags;
  const uint32_t* page_tags;
  int batch, num_kv_heads, head_dim, table_width, num_pages, n_max;
  int pages_per_unit;         // ceil(n_max / S) + 1: grid slots per unit
  bool head_layout, fp8;
};

// Compaction after eviction: the kept tokens of each unit, in list order, are
// rewritten from position 0 into the pages of a new table.
struct CompactArgs {
  const uint8_t* k_old;      // pools (the same allocations as k_new / v_new)
  const uint8_t* v_old;
  uint8_t* k_new;
  uint8_t* v_new;
  float* k_scale;            // FP8 only
  float* v_scale;
  const int32_t* block_table;  // old table
  const int32_t* lens;         // old lengths
  const int32_t* keep;         // [B][Hkv][keep_stride] positions to keep
  const int32_t* n_keep;       // lens' shape
  const int32_t* new_table;    // the old table's shape
  float* scores;               // nullptr or [P][Hkv_u][S]
  uint32_t* flags;             // nullptr or [B]
  int batch, num_kv_heads, head_dim, table_width, num_pages, keep_stride;
  int pages_per_unit;          // ceil(keep_stride / S): grid slots per unit
  bool head_layout, fp8;
};

// Pool slot of the V block of (page pid, KV head h).  The V block of a
// (page, head) is not stored at the same slot as its K block: K and V pools
// are separate allocations, commonly aligned alike, and a wave requests the K
// and V blocks of a page back to back; at equal offsets both requests fall in
// the same HBM bank (measured: about 5% of decode bandwidth lost).  SEQ layout
// with several heads: head h's V goes to head (h + 1) % Hkv's slot of the same
// page; otherwise page pid's V goes to page pid ^ 1's slot (pid itself when
// pid ^ 1 is past the pool).  A bijection, so every slot is still used once.
__host__ __device__ inline size_t v_block_slot(int pid, int h, int num_kv_heads, int num_pages,
                                               bool head_layout) {
  if (!head_layout && num_kv_heads > 1)
    return (size_t)pid * num_kv_heads + (h + 1 == num_kv_heads ? 0 : h + 1);
  const int q = pid ^ 1;
  const int p = q < num_pages ? q : pid;
  return head_layout ? (size_t)p : (size_t)p * num_kv_heads + h;
}

// Validation of v->batch sequences (v may be null) and up to two split plans
// (p0, p1 may be null), in one launch.
// Validation and split plans (either may be absent) in one launch; with `app`,
// a decode step's append runs in the same launch (step_prep_kernel).
hipError_t launch_prep(const ValidateArgs* v, const PlanArgs* p0, const PlanArgs* p1,
                       const AppendArgs* app, hipStream_t s);
hipError_t launch_attention(const AttnArgs& a, int head_dim, bool fp8, bool head_layout,
                            hipStream_t s);
hipError_t launch_reduce(const AttnArgs& a, int head_dim, bool head_layout, hipStream_t s);
hipError_t launch_append(const AppendArgs& a, hipStream_t s);
hipError_t launch_mass(const AttnArgs& a, int head_dim, bool fp8, bool head_layout, hipStream_t s);
hipError_t launch_compact(const CompactArgs& a, hipStream_t s);

}  // namespace pa
