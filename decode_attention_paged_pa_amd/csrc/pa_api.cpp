// C-ABI entry points of libpa: argument checks, partition choice, workspace
// sizing and kernel launches.  Declarations and contracts are in pa.h.
#include "pa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "pa_internal.h"

#define PA_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kVersion = 500;  // 0.5.0: a decode step in one call (pa_decode_step)

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_cache(const pa_cache_desc* c) {
  if (!c) return PA_ERR_INVALID_ARG;
  if (c->layout != PA_LAYOUT_SEQ && c->layout != PA_LAYOUT_HEAD) return PA_ERR_INVALID_ARG;
  if (c->kv_dtype != PA_KV_BF16 && c->kv_dtype != PA_KV_FP8_E4M3) return PA_ERR_INVALID_ARG;
  if (c->num_pages <= 0 || c->num_kv_heads <= 0) return PA_ERR_INVALID_ARG;
  if (c->page_size != pa::kPageSize) return PA_ERR_UNSUPPORTED;
  if (c->head_dim != 64 && c->head_dim != 128) return PA_ERR_UNSUPPORTED;
  // the kernels form page offsets with 32-bit page strides
  const int64_t esz = c->kv_dtype == PA_KV_FP8_E4M3 ? 1 : 2;
  if ((int64_t)c->num_kv_heads * c->page_size * c->head_dim * esz > INT32_MAX) return PA_ERR_UNSUPPORTED;
  if (!c->k_pages || !c->v_pages) return PA_ERR_INVALID_ARG;
  if (!aligned(c->k_pages, 256) || !aligned(c->v_pages, 256)) return PA_ERR_INVALID_ARG;
  if (c->kv_dtype == PA_KV_FP8_E4M3) {
    if (!c->k_scale || !c->v_scale) return PA_ERR_INVALID_ARG;
    if (!aligned(c->k_scale, 4) || !aligned(c->v_scale, 4)) return PA_ERR_INVALID_ARG;
  }
  return PA_OK;
}

int check_seq(const pa_seq_desc* s) {
  if (!s) return PA_ERR_INVALID_ARG;
  if (s->batch <= 0 || s->table_width <= 0) return PA_ERR_INVALID_ARG;
  if ((int64_t)s->table_width * pa::kPageSize > INT32_MAX) return PA_ERR_INVALID_ARG;
  if (!s->block_table || !s->lens) return PA_ERR_INVALID_ARG;
  if (!aligned(s->block_table, 4) || !aligned(s->lens, 4)) return PA_ERR_INVALID_ARG;
  if (s->expected_tags && !aligned(s->expected_tags, 4)) return PA_ERR_INVALID_ARG;
  return PA_OK;
}

int check_heads(const pa_cache_desc* c, int32_t num_q_heads, int32_t q_len = 1) {
  if (num_q_heads <= 0 || num_q_heads % c->num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (q_len < 1) return PA_ERR_INVALID_ARG;
  const int group = num_q_heads / c->num_kv_heads;
  if (group > pa::kMaxGroup || q_len > pa::kMaxQLen) return PA_ERR_UNSUPPORTED;
  if (q_len > 1 && group * q_len > pa::kMaxCols) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

size_t elem_bytes(const pa_cache_desc* c) { return c->kv_dtype == PA_KV_FP8_E4M3 ? 1 : 2; }

// Token partitioning of each unit: partitions are runs of chunk_pages pages.
// Automatic choice: about 2048 partitions at the table's capacity (two waves
// per SIMD on 256 compute units), 32 to 512 pages each.  A wave streams
// parts_per_wave consecutive partitions of its unit (writing one partial per
// partition): measured on MI355X, about 2048 long-running waves move the
// cache faster than 4096 shorter ones, so small partitions are grouped until
// the grid drops to that size.
constexpr int64_t kTargetWaves = 2048;
constexpr int64_t kSharedTargetGroups = 1536;   // prefill page-sharing workgroups: 2 rounds of 3 per CU

void choose_partitions(const pa_cache_desc* c, const pa_seq_desc* s, int32_t req,
                       int* chunk_pages, int* num_parts, int* parts_per_wave) {
  const int W = s->table_width;
  const int64_t units = (int64_t)s->batch * c->num_kv_heads;
  int cp;
  if (req > 0) {
    cp = (W + req - 1) / req;
  } else {
    int64_t x = (units * W + kTargetWaves - 1) / kTargetWaves;
    if (x < 32) x = 32;
    if (x > 512) x = 512;
    cp = (int)x;
  }
  if (cp > W) cp = W;
  if (cp < 1) cp = 1;
  const int parts = (W + cp - 1) / cp;
  int ppw = 1;  // at most 2: the attention kernel parks one finished partition per wave
  if (parts >= 2 && units * ((parts + 1) / 2) >= kTargetWaves) ppw = 2;
  *chunk_pages = cp;
  *num_parts = parts;
  if (parts_per_wave) *parts_per_wave = ppw;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// How a call splits each unit's pages.  Fixed: chunk_pages per partition,
// parts partitions (an explicit count, prefill, and tables of at most
// kPlanMinChunk pages).  Planned (automatic decode): plan_block picks the
// chunk on the device from the real lengths, for at most kPlanWaves waves of
// equal work; a plan holds at most max_pairs (group, partition) pairs.
#ifndef PA_PLAN_WAVES
#define PA_PLAN_WAVES 2048
#endif
#ifndef PA_PLAN_MIN_CHUNK
#define PA_PLAN_MIN_CHUNK 32
#endif
constexpr int64_t kPlanWaves = PA_PLAN_WAVES;      // waves of equal work the plan aims for
constexpr int kPlanMinChunk = PA_PLAN_MIN_CHUNK;   // pages; below this a wave's fixed costs weigh

struct Split {
  bool planned = false;
  int chunk_pages = 1, parts = 1, ppw = 1;
  int groups = 0, hpg = 1, max_pairs = 0;   // planned only
};

Split decode_split(const pa_cache_desc* c, const pa_seq_desc* s, int32_t req) {
  Split sp;
  if (req == 0 && s->table_width > kPlanMinChunk) {
    const bool head = c->layout == PA_LAYOUT_HEAD;
    sp.planned = true;
    sp.hpg = head ? 1 : c->num_kv_heads;
    sp.groups = head ? s->batch * c->num_kv_heads : s->batch;
    // pairs <= pages / chunk + groups, and chunk >= pages * hpg / kPlanWaves
    sp.max_pairs = (int)((kPlanWaves + sp.hpg - 1) / sp.hpg) + sp.groups;
    return sp;
  }
  choose_partitions(c, s, req, &sp.chunk_pages, &sp.parts, &sp.ppw);
  return sp;
}

void choose_prefill_partitions(const pa_cache_desc* c, const pa_seq_desc* s, int32_t hq,
                               int32_t q_len, int32_t req, int* chunk_pages, int* num_parts);

Split prefill_split(const pa_cache_desc* c, const pa_seq_desc* s, int32_t hq, int32_t q_len,
                    int32_t req) {
  Split sp;
  choose_prefill_partitions(c, s, hq, q_len, req, &sp.chunk_pages, &sp.parts);
  return sp;
}

// Partials: fixed partitions [B][T][Hq][Pn] (D floats, then (max, sum)) when
// Pn > 1; planned, [pair][head in group][T * G columns] plus the plan
// (int32: chunk, pair count, groups + 1 first pairs, the group of each pair).
// A scored decode also keeps the rows' final (max, sum) [B][Hq][2].
Split mass_split(const pa_cache_desc* c, const pa_seq_desc* s);

struct WorkspaceLayout {
  size_t part_o = 0, part_ml = 0, plan = 0, plan_group = 0, plan_rec = 0, row_ml = 0;
  size_t mass_plan = 0, mass_group = 0, unit_flags = 0, total = 0;
};

WorkspaceLayout workspace_layout(const pa_cache_desc* c, const pa_seq_desc* s, int32_t hq,
                                 int32_t q_len, const Split& sp, bool scored) {
  WorkspaceLayout w;
  size_t off = 0;
  if (sp.planned) {
    const size_t slots = (size_t)sp.max_pairs * sp.hpg * (hq / c->num_kv_heads) * q_len;
    w.part_o = off;
    off += align256(slots * c->head_dim * sizeof(float));
    w.part_ml = off;
    off += align256(slots * 2 * sizeof(float));
    w.plan = off;
    off += align256(((size_t)sp.groups + 3) * sizeof(int32_t));
    w.plan_group = off;
    off += align256((size_t)sp.max_pairs * sizeof(int32_t));
    w.plan_rec = off;
    off += align256((size_t)sp.max_pairs * 4 * sizeof(int32_t));
  } else if (sp.parts > 1) {
    const size_t rows = (size_t)s->batch * q_len * hq * sp.parts;
    w.part_o = off;
    off += align256(rows * c->head_dim * sizeof(float));
    w.part_ml = off;
    off += align256(rows * 2 * sizeof(float));
  }
  if (c->layout == PA_LAYOUT_HEAD) {   // the validation's word per unit
    w.unit_flags = off;
    off += align256((size_t)s->batch * c->num_kv_heads * sizeof(uint32_t));
  }
  if (scored) {
    w.row_ml = off;
    off += align256((size_t)s->batch * hq * 2 * sizeof(float));
    const Split ms = mass_split(c, s);
    w.mass_plan = off;
    off += align256(((size_t)ms.groups + 3) * sizeof(int32_t));
    w.mass_group = off;
    off += align256((size_t)ms.max_pairs * sizeof(int32_t));
  }
  w.total = off;
  return w;
}

size_t workspace_for(const pa_cache_desc* c, const pa_seq_desc* s, int32_t hq, int32_t q_len,
                     const Split& sp, bool scored = false) {
  return workspace_layout(c, s, hq, q_len, sp, scored).total;
}

// Eviction score pass: K-only streaming, one wave per run of 16 to kMassRun
// pages (the wave's LDS rows), from a length-balanced plan of its own aiming
// at kMassPlanWaves waves.
#ifndef PA_MASS_WAVES
#define PA_MASS_WAVES 4096
#endif
constexpr int kMassPlanWaves = PA_MASS_WAVES;
constexpr int kMassMinChunk = 16;

Split mass_split(const pa_cache_desc* c, const pa_seq_desc* s) {
  Split sp;
  const bool head = c->layout == PA_LAYOUT_HEAD;
  sp.planned = true;
  sp.hpg = head ? 1 : c->num_kv_heads;
  sp.groups = head ? s->batch * c->num_kv_heads : s->batch;
  // a fitting chunk gives at most target / hpg + groups pairs; the cap
  // (kMassRun pages) at most ceil(W / kMassRun) per group
  const int64_t fit = (kMassPlanWaves + sp.hpg - 1) / sp.hpg + sp.groups;
  const int64_t capped = (int64_t)sp.groups * ((s->table_width + pa::kMassRun - 1) / pa::kMassRun);
  sp.max_pairs = (int)(fit > capped ? fit : capped);
  return sp;
}

// Chunked prefill: a unit's G * T query columns go in blocks of kPrefillCols
// (32: four blocks per page-sharing workgroup), so there are far more waves
// than units; split-K is only needed when the grid would otherwise be small.
int prefill_col_blocks(const pa_cache_desc* c, int32_t hq, int32_t q_len) {
  const int64_t cols = (int64_t)(hq / c->num_kv_heads) * q_len;
  if (cols <= pa::kMaxCols) return 1;   // one multi-query wave holds the unit's columns
  return (int)((cols + pa::kPrefillCols - 1) / pa::kPrefillCols);
}

void choose_prefill_partitions(const pa_cache_desc* c, const pa_seq_desc* s, int32_t hq,
                               int32_t q_len, int32_t req, int* chunk_pages, int* num_parts) {
  const int W = s->table_width;
  int parts = req;
  if (req <= 0) {
    // Work items: waves of 64 columns; with the page-sharing kernel (blocks
    // of 32 columns), workgroups of kWaves blocks, aiming at two rounds of the
    // 3 resident per CU.  Measured on MI355X (512-token chunk over 0-30K
    // prefixes, 512 workgroups): 1, 2, 3, 4 and 6 partitions took 1346, 729,
    // 551, 738 and 573 us; the 2048-token chunk (2048 workgroups) is fastest
    // unsplit.
    const int64_t cb = prefill_col_blocks(c, hq, q_len);
    const bool shared = pa::kPrefillCols == 32 && cb > 1;
    const int64_t items = (int64_t)s->batch * c->num_kv_heads *
                          (shared ? (cb + pa::kWaves - 1) / pa::kWaves : cb);
    const int64_t target = shared ? kSharedTargetGroups : kTargetWaves;
    int64_t p = (target + items - 1) / items;
    const int64_t pmax = (W + 31) / 32;               // partitions of at least 32 pages
    parts = (int)(p < 1 ? 1 : (p > pmax ? pmax : p));
  }
  int cp = (W + parts - 1) / parts;
  if (cp > W) cp = W;
  if (cp < 1) cp = 1;
  *chunk_pages = cp;
  *num_parts = (W + cp - 1) / cp;
}

int check_prefill(const pa_cache_desc* c, const pa_seq_desc* s, int32_t hq, int32_t q_len) {
  if (hq <= 0 || hq % c->num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (hq / c->num_kv_heads > pa::kMaxGroup) return PA_ERR_UNSUPPORTED;
  if (q_len < 1 || (int64_t)q_len > (int64_t)s->table_width * pa::kPageSize) return PA_ERR_INVALID_ARG;
  if ((int64_t)s->batch * q_len * hq > INT32_MAX) return PA_ERR_INVALID_ARG;
  return PA_OK;
}

// Arguments of one planner workgroup (see plan_block): group lengths are the
// sequence's (SEQ) or the unit's (HEAD) entries of seq->lens.
pa::PlanArgs plan_args(const pa_seq_desc* seq, const Split& sp, char* plan, char* group,
                       int target_waves, int min_chunk, int max_chunk) {
  pa::PlanArgs p{};
  p.lens = seq->lens;
  p.plan = reinterpret_cast<int32_t*>(plan);
  p.plan_group = reinterpret_cast<int32_t*>(group);
  p.num_groups = sp.groups;
  p.heads_per_group = sp.hpg;
  p.table_width = seq->table_width;
  p.max_pairs = sp.max_pairs;
  p.target_waves = target_waves;
  p.min_chunk = min_chunk;
  p.max_chunk = max_chunk;
  return p;
}

// Arguments of an append of n_new[u] tokens (at most n_max) at positions
// lens_old[u]... through seq's table; k_new / v_new are [B][Hkv][n_max][D].
int append_args(const pa_cache_desc* cache, const pa_seq_desc* seq, const int32_t* lens_old,
                const int32_t* n_new, int32_t n_max, const uint16_t* k_new,
                const uint16_t* v_new, pa::AppendArgs* out) {
  if (!lens_old || !aligned(lens_old, 4) || !n_new || !aligned(n_new, 4) || n_max < 0)
    return PA_ERR_INVALID_ARG;
  if (n_max > 0 && (!k_new || !v_new || !aligned(k_new, 2) || !aligned(v_new, 2)))
    return PA_ERR_INVALID_ARG;
  pa::AppendArgs a{};
  a.k_pages = static_cast<uint8_t*>(cache->k_pages);
  a.v_pages = static_cast<uint8_t*>(cache->v_pages);
  a.k_scale = cache->k_scale;
  a.v_scale = cache->v_scale;
  a.block_table = seq->block_table;
  a.lens_old = lens_old;
  a.n_new = n_new;
  a.k_new = k_new;
  a.v_new = v_new;
  if (seq->expected_tags) {   // writes gated on the tags of the pages they land in
    if (!cache->page_tags || !aligned(cache->page_tags, 4)) return PA_ERR_INVALID_ARG;
    a.expected_tags = seq->expected_tags;
    a.page_tags = cache->page_tags;
  }
  a.batch = seq->batch;
  a.num_kv_heads = cache->num_kv_heads;
  a.head_dim = cache->head_dim;
  a.table_width = seq->table_width;
  a.num_pages = cache->num_pages;
  a.n_max = n_max;
  a.pages_per_unit = n_max == 0 ? 0 : (n_max + pa::kPageSize - 1) / pa::kPageSize + 1;
  a.head_layout = cache->layout == PA_LAYOUT_HEAD;
  a.fp8 = cache->kv_dtype == PA_KV_FP8_E4M3;
  if ((int64_t)a.batch * a.num_kv_heads * a.pages_per_unit > INT32_MAX) return PA_ERR_INVALID_ARG;
  *out = a;
  return PA_OK;
}

int decode_impl(const pa_cache_desc* cache, const pa_seq_desc* seq, int32_t num_q_heads,
                int32_t q_len, const uint16_t* q, uint16_t* out, float softmax_scale,
                int32_t num_partitions, uint32_t* flags, void* workspace, size_t workspace_bytes,
                hipStream_t stream, pa_event_t const* events, float* scores = nullptr,
                bool prefill = false, const pa::AppendArgs* app = nullptr) {
  int rc;
  if ((rc = check_cache(cache)) != PA_OK) return rc;
  if ((rc = check_seq(seq)) != PA_OK) return rc;
  if (prefill) {
    if ((rc = check_prefill(cache, seq, num_q_heads, q_len)) != PA_OK) return rc;
  } else if ((rc = check_heads(cache, num_q_heads, q_len)) != PA_OK) {
    return rc;
  }
  if (!q || !out || !aligned(q, 16) || !aligned(out, 16)) return PA_ERR_INVALID_ARG;
  if (!std::isfinite(softmax_scale)) return PA_ERR_INVALID_ARG;
  if (num_partitions < 0) return PA_ERR_INVALID_ARG;
  if (seq->expected_tags && (!flags || !cache->page_tags)) return PA_ERR_INVALID_ARG;
  if (flags && !aligned(flags, 4)) return PA_ERR_INVALID_ARG;
  if (scores && (q_len != 1 || !aligned(scores, 4))) return PA_ERR_INVALID_ARG;
  const Split sp = prefill ? prefill_split(cache, seq, num_q_heads, q_len, num_partitions)
                           : decode_split(cache, seq, num_partitions);
  const WorkspaceLayout wl =
      workspace_layout(cache, seq, num_q_heads, q_len, sp, scores != nullptr);
  const size_t need = wl.total;
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256)))
    return PA_ERR_WORKSPACE;
  const bool head = cache->layout == PA_LAYOUT_HEAD;
  const bool fp8 = cache->kv_dtype == PA_KV_FP8_E4M3;

  auto rec = [&](int i) {
    if (events && events[i]) (void)hipEventRecord(reinterpret_cast<hipEvent_t>(events[i]), stream);
  };

  rec(0);
  char* ws = static_cast<char*>(workspace);
  // HEAD layout: one validation workgroup and word per unit; the decode ORs a
  // sequence's words and its last kernel writes flags[b]
  const bool per_unit = flags && head;
  uint32_t* unit_flags = per_unit ? reinterpret_cast<uint32_t*>(ws + wl.unit_flags) : nullptr;
  pa::ValidateArgs v{};
  if (flags) {
    v.block_table = seq->block_table;
    v.lens = seq->lens;
    v.expected_tags = seq->expected_tags;
    v.page_tags = cache->page_tags;
    v.flags = per_unit ? unit_flags : flags;
    v.batch = seq->batch;
    v.num_kv_heads = cache->num_kv_heads;
    v.table_width = seq->table_width;
    v.num_pages = cache->num_pages;
    v.head_layout = head;
    v.per_unit = per_unit;
    v.rows = per_unit ? seq->batch * cache->num_kv_heads : seq->batch;
  }
  // the decode's split (automatic) and the score pass's split (scored decode)
  const Split ms = scores ? mass_split(cache, seq) : Split{};
  pa::PlanArgs pl = plan_args(seq, sp, ws + wl.plan, ws + wl.plan_group, (int)kPlanWaves,
                                    kPlanMinChunk, seq->table_width);
  if (sp.planned) pl.plan_rec = reinterpret_cast<int32_t*>(ws + wl.plan_rec);
  const pa::PlanArgs pm = plan_args(seq, ms, ws + wl.mass_plan, ws + wl.mass_group,
                                    kMassPlanWaves, kMassMinChunk, pa::kMassRun);
  if (pa::launch_prep(flags ? &v : nullptr, sp.planned ? &pl : nullptr, scores ? &pm : nullptr,
                      app, stream) != hipSuccess)
    return PA_ERR_LAUNCH;
  rec(1);

  pa::AttnArgs a{};
  a.k_pages = static_cast<const uint8_t*>(cache->k_pages);
  a.v_pages = static_cast<const uint8_t*>(cache->v_pages);
  a.k_scale = cache->k_scale;
  a.v_scale = cache->v_scale;
  a.block_table = seq->block_table;
  a.lens = seq->lens;
  a.flags = flags;
  a.unit_flags = unit_flags;
  a.flags_out = flags;
  a.q = q;
  a.out = out;
  if (sp.planned || sp.parts > 1) {
    a.part_o = reinterpret_cast<float*>(ws + wl.part_o);
    a.part_ml = reinterpret_cast<float*>(ws + wl.part_ml);
  }
  if (sp.planned) {
    a.plan = reinterpret_cast<const int32_t*>(ws + wl.plan);
    a.plan_group = reinterpret_cast<const int32_t*>(ws + wl.plan_group);
    a.plan_rec = reinterpret_cast<const int32_t*>(ws + wl.plan_rec);
    a.max_pairs = sp.max_pairs;
  }
  if (scores) a.row_ml = reinterpret_cast<float*>(ws + wl.row_ml);
  a.batch = seq->batch;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = cache->num_kv_heads;
  a.group = num_q_heads / cache->num_kv_heads;
  a.q_len = q_len;
  a.col_blocks = prefill ? prefill_col_blocks(cache, num_q_heads, q_len) : 1;
  a.table_width = seq->table_width;
  a.num_pages = cache->num_pages;
  a.chunk_pages = sp.chunk_pages;
  a.num_parts = sp.parts;
  a.parts_per_wave = sp.ppw;
  // XCD-aware workgroup order needs whole groups of 4 heads; the SEQ layout
  // gains most from it (the heads of a page share its blocks and scales).  A
  // planned HEAD split has one head per pair and keeps the plain order.
  a.xcd_order = (cache->num_kv_heads % pa::kWaves == 0 && a.col_blocks == 1 &&
                 !(sp.planned && head)) ? 1 : 0;
#ifdef PA_NO_XCD_ORDER
  a.xcd_order = 0;
#endif
  a.score_scale_log2 = (float)((double)softmax_scale * 1.4426950408889634);
  const bool reduce = sp.planned || sp.parts > 1;
  a.write_flags = (per_unit && !reduce) ? 1 : 0;   // the decode's last kernel writes flags[b]
  if (pa::launch_attention(a, cache->head_dim, fp8, head, stream) != hipSuccess)
    return PA_ERR_LAUNCH;
  rec(2);
  if (reduce) {
    a.write_flags = per_unit ? 1 : 0;
    if (pa::launch_reduce(a, cache->head_dim, head, stream) != hipSuccess) return PA_ERR_LAUNCH;
  }
  if (scores) {   // second pass: K again, with the rows' final (max, sum)
    pa::AttnArgs m = a;
    m.scores = scores;
    m.plan = reinterpret_cast<const int32_t*>(ws + wl.mass_plan);
    m.plan_group = reinterpret_cast<const int32_t*>(ws + wl.mass_group);
    m.max_pairs = ms.max_pairs;
    if (pa::launch_mass(m, cache->head_dim, fp8, head, stream) != hipSuccess) return PA_ERR_LAUNCH;
  }
  rec(3);
  return PA_OK;
}

}  // namespace

PA_API size_t pa_pool_bytes(const pa_cache_desc* c) {
  if (!c || c->num_pages <= 0 || c->num_kv_heads <= 0 || c->page_size <= 0 || c->head_dim <= 0)
    return 0;
  if (c->kv_dtype != PA_KV_BF16 && c->kv_dtype != PA_KV_FP8_E4M3) return 0;
  const size_t heads = c->layout == PA_LAYOUT_SEQ ? (size_t)c->num_kv_heads : 1;
  return (size_t)c->num_pages * heads * c->page_size * c->head_dim * elem_bytes(c);
}

PA_API int pa_cache_append(const pa_cache_desc* cache, const pa_seq_desc* seq,
                           const int32_t* n_new, int32_t n_max, const uint16_t* k_new,
                           const uint16_t* v_new, uint32_t* flags, pa_stream_t stream) {
  int rc;
  if ((rc = check_cache(cache)) != PA_OK) return rc;
  if ((rc = check_seq(seq)) != PA_OK) return rc;
  if (n_max == 0 && !flags && n_new && aligned(n_new, 4)) return PA_OK;
  pa::AppendArgs a{};
  if ((rc = append_args(cache, seq, seq->lens, n_new, n_max, k_new, v_new, &a)) != PA_OK)
    return rc;
  if (flags && !aligned(flags, 4)) return PA_ERR_INVALID_ARG;
  a.flags = flags;
  if (pa::launch_append(a, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return PA_ERR_LAUNCH;
  return PA_OK;
}

PA_API size_t pa_decode_workspace_bytes(const pa_cache_desc* cache, const pa_seq_desc* seq,
                                        int32_t num_q_heads, int32_t num_partitions) {
  if (check_cache(cache) != PA_OK || check_seq(seq) != PA_OK ||
      check_heads(cache, num_q_heads) != PA_OK || num_partitions < 0)
    return (size_t)-1;
  return workspace_for(cache, seq, num_q_heads, 1, decode_split(cache, seq, num_partitions));
}

PA_API size_t pa_decode_multi_workspace_bytes(const pa_cache_desc* cache, const pa_seq_desc* seq,
                                              int32_t num_q_heads, int32_t q_len,
                                              int32_t num_partitions) {
  if (check_cache(cache) != PA_OK || check_seq(seq) != PA_OK ||
      check_heads(cache, num_q_heads, q_len) != PA_OK || num_partitions < 0)
    return (size_t)-1;
  return workspace_for(cache, seq, num_q_heads, q_len, decode_split(cache, seq, num_partitions));
}

PA_API int pa_decode_num_partitions(const pa_cache_desc* cache, const pa_seq_desc* seq,
                                    int32_t num_q_heads, int32_t num_partitions) {
  int rc;
  if ((rc = check_cache(cache)) != PA_OK) return rc;
  if ((rc = check_seq(seq)) != PA_OK) return rc;
  if ((rc = check_heads(cache, num_q_heads)) != PA_OK) return rc;
  if (num_partitions < 0) return PA_ERR_INVALID_ARG;
  const Split sp = decode_split(cache, seq, num_partitions);
  return sp.planned ? 0 : sp.parts;
}

PA_API int pa_decode(const pa_cache_desc* cache, const pa_seq_desc* seq, int32_t num_q_heads,
                     const uint16_t* q, uint16_t* out, float softmax_scale,
                     int32_t num_partitions, uint32_t* flags, void* workspace,
                     size_t workspace_bytes, pa_stream_t stream) {
  return decode_impl(cache, seq, num_q_heads, 1, q, out, softmax_scale, num_partitions, flags,
                     workspace, workspace_bytes, reinterpret_cast<hipStream_t>(stream), nullptr);
}

// ---------------------------------------------- pa_decode_noalloc's scratch
// A static device array in place of the caller's workspace, for callers that
// cannot allocate.  In host code `scratch` names a host-side stand-in, not
// the device array: its device address (one per GPU, each GPU holding its
// own copy) comes from hipGetSymbolAddress, taken once per device with that
// device current and kept in scratch_ptr[]; only that address is ever passed
// to a kernel.
namespace {
constexpr size_t kScratchBytes = PA_NOALLOC_SCRATCH_BYTES;
constexpr int kScratchDevices = 64;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
std::mutex scratch_mu;
void* scratch_ptr[kScratchDevices] = {};

// The current device's scratch address; the stream must belong to that device.
int device_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return PA_ERR_LAUNCH;
  if (dev >= kScratchDevices) return PA_ERR_UNSUPPORTED;
  if (stream) {
    hipDevice_t sd = -1;
    if (hipStreamGetDevice(stream, &sd) != hipSuccess || sd != dev) return PA_ERR_INVALID_ARG;
  }
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PA_ERR_LAUNCH;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return PA_OK;
}
}  // namespace

PA_API int pa_decode_noalloc(const pa_cache_desc* cache, const pa_seq_desc* seq,
                             int32_t num_q_heads, const uint16_t* q, uint16_t* out,
                             float softmax_scale, int32_t num_partitions, uint32_t* flags,
                             pa_stream_t stream) {
  const size_t need = pa_decode_workspace_bytes(cache, seq, num_q_heads, num_partitions);
  if (need == (size_t)-1) {   // the argument errors, as pa_decode reports them
    return decode_impl(cache, seq, num_q_heads, 1, q, out, softmax_scale, num_partitions, flags,
                       nullptr, 0, reinterpret_cast<hipStream_t>(stream), nullptr);
  }
  if (need > kScratchBytes) return PA_ERR_SCRATCH;
  void* ws = nullptr;
  const int rc = device_scratch(reinterpret_cast<hipStream_t>(stream), &ws);
  if (rc != PA_OK) return rc;
  return decode_impl(cache, seq, num_q_heads, 1, q, out, softmax_scale, num_partitions, flags,
                     ws, kScratchBytes, reinterpret_cast<hipStream_t>(stream), nullptr);
}

PA_API int pa_decode_timed(const pa_cache_desc* cache, const pa_seq_desc* seq,
                           int32_t num_q_heads, const uint16_t* q, uint16_t* out,
                           float softmax_scale, int32_t num_partitions, uint32_t* flags,
                           void* workspace, size_t workspace_bytes, pa_stream_t stream,
                           pa_event_t const events[4]) {
  return decode_impl(cache, seq, num_q_heads, 1, q, out, softmax_scale, num_partitions, flags,
                     workspace, workspace_bytes, reinterpret_cast<hipStream_t>(stream), events);
}

PA_API size_t pa_decode_scored_workspace_bytes(const pa_cache_desc* cache, const pa_seq_desc* seq,
                                               int32_t num_q_heads, int32_t num_partitions) {
  if (check_cache(cache) != PA_OK || check_seq(seq) != PA_OK ||
      check_heads(cache, num_q_heads) != PA_OK || num_partitions < 0)
    return (size_t)-1;
  return workspace_for(cache, seq, num_q_heads, 1, decode_split(cache, seq, num_partitions), true);
}

PA_API int pa_decode_scored(const pa_cache_desc* cache, const pa_seq_desc* seq,
                            int32_t num_q_heads, const uint16_t* q, uint16_t* out,
                            float softmax_scale, int32_t num_partitions, uint32_t* flags,
                            float* scores, void* workspace, size_t workspace_bytes,
                            pa_stream_t stream) {
  if (!scores) return PA_ERR_INVALID_ARG;
  return decode_impl(cache, seq, num_q_heads, 1, q, out, softmax_scale, num_partitions, flags,
                     workspace, workspace_bytes, reinterpret_cast<hipStream_t>(stream), nullptr,
                     scores);
}

PA_API int pa_decode_scored_timed(const pa_cache_desc* cache, const pa_seq_desc* seq,
                                  int32_t num_q_heads, const uint16_t* q, uint16_t* out,
                                  float softmax_scale, int32_t num_partitions, uint32_t* flags,
                                  float* scores, void* workspace, size_t workspace_bytes,
                                  pa_stream_t stream, pa_event_t const events[4]) {
  if (!scores) return PA_ERR_INVALID_ARG;
  return decode_impl(cache, seq, num_q_heads, 1, q, out, softmax_scale, num_partitions, flags,
                     workspace, workspace_bytes, reinterpret_cast<hipStream_t>(stream), events,
                     scores);
}

PA_API int pa_cache_compact(const pa_cache_desc* cache, const pa_seq_desc* seq,
                            const int32_t* keep, int32_t keep_stride, const int32_t* n_keep,
                            const int32_t* new_table, float* scores, uint32_t* flags,
                            pa_stream_t stream) {
  int rc;
  if ((rc = check_cache(cache)) != PA_OK) return rc;
  if ((rc = check_seq(seq)) != PA_OK) return rc;
  if (keep_stride <= 0 || !keep || !n_keep || !new_table) return PA_ERR_INVALID_ARG;
  if (!aligned(keep, 4) || !aligned(n_keep, 4) || !aligned(new_table, 4)) return PA_ERR_INVALID_ARG;
  if ((scores && !aligned(scores, 4)) || (flags && !aligned(flags, 4))) return PA_ERR_INVALID_ARG;
  pa::CompactArgs a{};
  a.k_old = static_cast<const uint8_t*>(cache->k_pages);
  a.v_old = static_cast<const uint8_t*>(cache->v_pages);
  a.k_new = static_cast<uint8_t*>(cache->k_pages);
  a.v_new = static_cast<uint8_t*>(cache->v_pages);
  a.k_scale = cache->k_scale;
  a.v_scale = cache->v_scale;
  a.block_table = seq->block_table;
  a.lens = seq->lens;
  a.keep = keep;
  a.n_keep = n_keep;
  a.new_table = new_table;
  a.scores = scores;
  a.flags = flags;
  a.batch = seq->batch;
  a.num_kv_heads = cache->num_kv_heads;
  a.head_dim = cache->head_dim;
  a.table_width = seq->table_width;
  a.num_pages = cache->num_pages;
  a.keep_stride = keep_stride;
  a.pages_per_unit = (keep_stride + pa::kPageSize - 1) / pa::kPageSize;
  a.head_layout = cache->layout == PA_LAYOUT_HEAD;
  a.fp8 = cache->kv_dtype == PA_KV_FP8_E4M3;
  const int64_t grid = (int64_t)a.batch * a.num_kv_heads * a.pages_per_unit;
  if (grid > INT32_MAX) return PA_ERR_INVALID_ARG;
  if (pa::launch_compact(a, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return PA_ERR_LAUNCH;
  return PA_OK;
}

PA_API size_t pa_prefill_workspace_bytes(const pa_cache_desc* cache, const pa_seq_desc* seq,
                                         int32_t num_q_heads, int32_t chunk_len,
                                         int32_t num_partitions) {
  if (check_cache(cache) != PA_OK || check_seq(seq) != PA_OK ||
      check_prefill(cache, seq, num_q_heads, chunk_len) != PA_OK || num_partitions < 0)
    return (size_t)-1;
  return workspace_for(cache, seq, num_q_heads, chunk_len,
                       prefill_split(cache, seq, num_q_heads, chunk_len, num_partitions));
}

PA_API int pa_prefill_num_partitions(const pa_cache_desc* cache, const pa_seq_desc* seq,
                                     int32_t num_q_heads, int32_t chunk_len,
                                     int32_t num_partitions) {
  int rc;
  if ((rc = check_cache(cache)) != PA_OK) return rc;
  if ((rc = check_seq(seq)) != PA_OK) return rc;
  if ((rc = check_prefill(cache, seq, num_q_heads, chunk_len)) != PA_OK) return rc;
  if (num_partitions < 0) return PA_ERR_INVALID_ARG;
  int cp, parts;
  choose_prefill_partitions(cache, seq, num_q_heads, chunk_len, num_partitions, &cp, &parts);
  return parts;
}

PA_API int pa_prefill(const pa_cache_desc* cache, const pa_seq_desc* seq, int32_t num_q_heads,
                      int32_t chunk_len, const uint16_t* q, uint16_t* out, float softmax_scale,
                      int32_t num_partitions, uint32_t* flags, void* workspace,
                      size_t workspace_bytes, pa_stream_t stream) {
  return decode_impl(cache, seq, num_q_heads, chunk_len, q, out, softmax_scale, num_partitions,
                     flags, workspace, workspace_bytes, reinterpret_cast<hipStream_t>(stream),
                     nullptr, nullptr, true);
}

PA_API int pa_prefill_timed(const pa_cache_desc* cache, const pa_seq_desc* seq,
                            int32_t num_q_heads, int32_t chunk_len, const uint16_t* q,
                            uint16_t* out, float softmax_scale, int32_t num_partitions,
                            uint32_t* flags, void* workspace, size_t workspace_bytes,
                            pa_stream_t stream, pa_event_t const events[4]) {
  return decode_impl(cache, seq, num_q_heads, chunk_len, q, out, softmax_scale, num_partitions,
                     flags, workspace, workspace_bytes, reinterpret_cast<hipStream_t>(stream),
                     events, nullptr, true);
}

PA_API int pa_decode_multi(const pa_cache_desc* cache, const pa_seq_desc* seq,
                           int32_t num_q_heads, int32_t q_len, const uint16_t* q, uint16_t* out,
                           float softmax_scale, int32_t num_partitions, uint32_t* flags,
                           void* workspace, size_t workspace_bytes, pa_stream_t stream) {
  return decode_impl(cache, seq, num_q_heads, q_len, q, out, softmax_scale, num_partitions, flags,
                     workspace, workspace_bytes, reinterpret_cast<hipStream_t>(stream), nullptr);
}

PA_API int pa_decode_multi_timed(const pa_cache_desc* cache, const pa_seq_desc* seq,
                                 int32_t num_q_heads, int32_t q_len, const uint16_t* q,
                                 uint16_t* out, float softmax_scale, int32_t num_partitions,
                                 uint32_t* flags, void* workspace, size_t workspace_bytes,
                                 pa_stream_t stream, pa_event_t const events[4]) {
  return decode_impl(cache, seq, num_q_heads, q_len, q, out, softmax_scale, num_partitions, flags,
                     workspace, workspace_bytes, reinterpret_cast<hipStream_t>(stream), events);
}

namespace {
int step_impl(const pa_cache_desc* cache, const pa_seq_desc* seq, const int32_t* lens_old,
              const int32_t* n_new, int32_t n_max, const uint16_t* k_new, const uint16_t* v_new,
              int32_t num_q_heads, int32_t q_len, const uint16_t* q, uint16_t* out,
              float softmax_scale, int32_t num_partitions, uint32_t* flags, void* workspace,
              size_t workspace_bytes, pa_stream_t stream, pa_event_t const* events) {
  int rc;
  if ((rc = check_cache(cache)) != PA_OK) return rc;
  if ((rc = check_seq(seq)) != PA_OK) return rc;
  pa::AppendArgs app{};
  if ((rc = append_args(cache, seq, lens_old, n_new, n_max, k_new, v_new, &app)) != PA_OK)
    return rc;
  return decode_impl(cache, seq, num_q_heads, q_len, q, out, softmax_scale, num_partitions, flags,
                     workspace, workspace_bytes, reinterpret_cast<hipStream_t>(stream), events,
                     nullptr, false, n_max > 0 ? &app : nullptr);
}
}  // namespace

PA_API int pa_decode_step(const pa_cache_desc* cache, const pa_seq_desc* seq,
                          const int32_t* lens_old, const int32_t* n_new, int32_t n_max,
                          const uint16_t* k_new, const uint16_t* v_new, int32_t num_q_heads,
                          int32_t q_len, const uint16_t* q, uint16_t* out, float softmax_scale,
                          int32_t num_partitions, uint32_t* flags, void* workspace,
                          size_t workspace_bytes, pa_stream_t stream) {
  return step_impl(cache, seq, lens_old, n_new, n_max, k_new, v_new, num_q_heads, q_len, q, out,
                   softmax_scale, num_partitions, flags, workspace, workspace_bytes, stream,
                   nullptr);
}

PA_API int pa_decode_step_timed(const pa_cache_desc* cache, const pa_seq_desc* seq,
                                const int32_t* lens_old, const int32_t* n_new, int32_t n_max,
                                const uint16_t* k_new, const uint16_t* v_new,
                                int32_t num_q_heads, int32_t q_len, const uint16_t* q,
                                uint16_t* out, float softmax_scale, int32_t num_partitions,
                                uint32_t* flags, void* workspace, size_t workspace_bytes,
                                pa_stream_t stream, pa_event_t const events[4]) {
  return step_impl(cache, seq, lens_old, n_new, n_max, k_new, v_new, num_q_heads, q_len, q, out,
                   softmax_scale, num_partitions, flags, workspace, workspace_bytes, stream,
                   events);
}

PA_API const char* pa_strerror(int code) {
  switch (code) {
    case PA_OK: return "success";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED:
      return "unsupported shape (page_size 16, head_dim 64/128, group <= 16, q_len <= 8, "
             "group * q_len <= 64)";
    case PA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case PA_ERR_LAUNCH: return "kernel launch failed";
    case PA_ERR_SCRATCH:
      return "the call needs more scratch than pa_decode_noalloc's static buffer holds "
             "(PA_NOALLOC_SCRATCH_BYTES); use pa_decode with a workspace";
    default: return "unknown error code";
  }
}

PA_API int pa_version(void) { return kVersion; }
