/*
 * crosscu — split-KV decode attention for AMD Instinct MI355X (gfx950).
 *
 * Each decode query token attends over its own sequence's paged KV cache:
 *   out = softmax(scale * q K^T) V,   lse = log sum exp(scale * q K^T).
 * The total KV work of a batch is cut Stream-K style into one equal chunk per
 * compute unit and run as a single persistent wave (CSDN Q&A on waves and
 * FlashMLA's Stream-K, "Summary").  Pieces of one sequence that land on
 * different compute units are merged just in time inside the same kernel by
 * the piece that finishes last (MeldKernel summary, "Core method": just-in-time
 * reduction instead of an HBM round trip and a separate reduction kernel).
 * The mapping is chosen at run time from the real sequence lengths and the
 * hardware shape (same summary, "Core method"; GLM-5.2 decode article, MegaRTP
 * design: only the host plan is rebuilt when lengths change).
 *
 * Conventions for every call below
 *  - Return value: CC_OK (0) or a negative CC_ERR_* code.  cc_last_error()
 *    returns a thread-local message for the last failing call of the thread.
 *  - Ownership: every buffer belongs to the caller.  Nothing is allocated per
 *    call and no pointer is retained after a call returns.
 *  - Host vs device: arguments documented "host" are read on the CPU during
 *    the call; "device" pointers must be device memory of the current HIP
 *    device and are only read/written by work enqueued on `stream`.
 *  - Streams: `stream` is a hipStream_t (NULL = the default stream).  Device
 *    work is enqueued asynchronously; no call synchronises unless stated.
 *  - No C++ exception crosses this interface.
 */
#ifndef CROSSCU_H
#define CROSSCU_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ codes */
enum {
  CC_OK = 0,
  CC_ERR_INVALID = -1,      /* null pointer, bad size or shape                  */
  CC_ERR_UNSUPPORTED = -2,  /* valid problem the kernels do not implement        */
  CC_ERR_BUFFER = -3,       /* caller buffer too small                           */
  CC_ERR_PLAN = -4,         /* plan blob malformed or built for another problem  */
  CC_ERR_PAGE = -5,         /* block_table entry outside [0, num_pages)          */
  CC_ERR_HIP = -6,          /* a HIP runtime call failed                         */
  CC_ERR_DEVICE_DATA = -7   /* cc_workspace_check: the device saw bad data       */
};

/* Attention forms.
 *  GQA:        separate K and V caches, Hkv heads, G = Hq / Hkv query heads
 *              per KV head; query head h reads KV head h / G; one query token.
 *  MLA:        one latent cache row of head_dim_qk columns per token serves as
 *              K; its first head_dim_v columns are V; Hkv = 1; one query token.
 *  MLA_SPARSE: as MLA, but query token t of request b attends only to the
 *              topk cache positions indices[b][t][0..topk).                    */
enum { CC_MODE_GQA = 0, CC_MODE_MLA = 1, CC_MODE_MLA_SPARSE = 2, CC_MODE_MOE = 3 /* cc_moe_* */ };

/* Page layouts of the GQA K and V caches (MLA caches have one head: both are
 * [num_pages][page_size][head_dim_qk]).
 *  NHD: [num_pages][page_size][num_kv_heads][head_dim]  token-major pages
 *  HND: [num_pages][num_kv_heads][page_size][head_dim]  head-major pages     */
enum { CC_KV_NHD = 0, CC_KV_HND = 1 };

/* How a plan divides the work.
 *  STREAMK:   the work is cut into num_cus equal contiguous chunks (one per
 *             compute unit, one wave); a sequence may be split.  What is cut
 *             evenly is the cost of the work: one per KV tile plus
 *             cc_plan_opts.unit_cost per non-empty unit (the fixed work of
 *             starting and finishing it).  Units are laid out in order, each
 *             unit's cost first, and a tile goes to the chunk whose cost range
 *             holds its starting position.  With unit_cost = 0 this is the
 *             plain equal split of the tile count: chunk k takes
 *             floor(N / C) tiles, one more for k < N mod C (CSDN Q&A on
 *             waves and FlashMLA's Stream-K, "Summary"; GLM-5.2 decode
 *             article, MegaRTP design: 732 tasks over 148 workers give 140
 *             workers 5 tasks and 8 workers 4).
 *  PER_UNIT:  one worker per unit (query heads sharing one K/V stream), no
 *             split — the classic one-workgroup-per-(sequence, head) launch. */
/*  STREAMK_DP: (cc_moe_plan only) the data-parallel + Stream-K form of the
 *             same equal split: the first D C units go whole, unit r C + k to
 *             chunk k in round r (so units computed at the same time are
 *             neighbours and share operand tiles in cache), and the remaining
 *             U - D C units are split as STREAMK splits them.  With
 *             R = U mod C: R = 0 or 4 R >= 3 C runs every unit whole (the
 *             last round's units on chunks 0 .. R - 1); 2 R >= C splits the
 *             remainder alone (D = U div C); a smaller remainder takes the
 *             last whole round with it (D = U div C - 1).  Each chunk's share
 *             of a split region is at least half a unit, so a split unit has
 *             at most three pieces at unit cost 0.  Every chunk gets the same
 *             work to within one tile.                                     */
enum { CC_POLICY_STREAMK = 0, CC_POLICY_PER_UNIT = 1, CC_POLICY_STREAMK_DP = 2 };

/* Unit costs (in tiles) measured for this library's kernels: a GQA unit's
 * start and finish cost about one 32-token tile, a 128-head MLA unit's (its
 * queries loaded, its 128 KiB partial written and published) about six.  They
 * are tuning values of these kernels, not part of the method; 0 gives the
 * pages' equal tile split. */
#define CC_UNIT_COST_GQA 1
#define CC_UNIT_COST_MLA 6

/* Reduction of split units inside cc_decode_variant.
 *  FUSED:          the last piece of a unit to finish merges the partials in
 *                  the same kernel (a per-unit arrival counter decides).
 *  SPLIT_COMBINE:  every piece writes its partial; a second kernel merges.  */
enum { CC_REDUCE_FUSED = 0, CC_REDUCE_SPLIT_COMBINE = 1 };

/* Problem shape.  Layouts (row-major, innermost last):
 *   q            bf16  [batch][q_tokens][num_q_heads][head_dim_qk]
 *   k_cache      bf16  [num_pages][page_size][num_kv_heads][head_dim_qk] (NHD)
 *                   or [num_pages][num_kv_heads][page_size][head_dim_qk] (HND)
 *   v_cache      bf16  as k_cache with head_dim_v (GQA only)
 *   block_table  int32 [batch][max_pages_per_seq]; token j of sequence b lives
 *                in page block_table[b][j / page_size], slot j % page_size.
 *                The slots of a sequence's last page past its length may hold
 *                any bits, NaN and Inf included: the kernels may read them
 *                (whole 32-token blocks inside a page) but never use them.
 *   seqlens      int32 [batch], each >= 0 (>= topk for MLA_SPARSE); a sequence
 *                with no cached tokens gets out = 0 and lse = -inf, the
 *                neutral element of the log-sum-exp merge
 *   indices      int32 [batch][q_tokens][topk] (MLA_SPARSE), distinct
 *                positions in [0, seqlens[b])
 *   out          fp32  [batch][q_tokens][num_q_heads][head_dim_v]
 *   lse          fp32  [batch][q_tokens][num_q_heads], natural log           */
typedef struct cc_problem {
  int32_t mode;
  int32_t batch;
  int32_t q_tokens;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim_qk;
  int32_t head_dim_v;
  int32_t page_size;
  int32_t max_pages_per_seq;
  int32_t num_pages;
  int32_t topk;             /* MLA_SPARSE only, else 0 */
  int32_t kv_layout;        /* CC_KV_NHD or CC_KV_HND */
  float softmax_scale;
} cc_problem;

/* Plan knobs.  num_cus / num_xcds: compute units and XCDs to plan for (see
 * cc_device_query).  tile_tokens: the cost unit of the equal split (any
 * value >= 1 plans; cc_decode needs a multiple of 32).  heads_per_unit: query
 * heads processed together on one K/V stream (divides Hq / Hkv; cc_decode's
 * GQA kernel needs Hq / Hkv, its MLA kernels need 128: all heads of a query
 * token form one unit, so each latent row is read once per query token).
 * policy: CC_POLICY_*.  unit_cost: CC_POLICY_STREAMK's cost of a unit in
 * tiles, >= 0 (0: the equal tile split; see CC_UNIT_COST_*).               */
typedef struct cc_plan_opts {
  int32_t num_cus;
  int32_t num_xcds;
  int32_t tile_tokens;
  int32_t heads_per_unit;
  int32_t policy;
  int32_t unit_cost;
} cc_plan_opts;

/* Library version (major * 10000 + minor * 100 + patch). */
int cc_version(void);

/* Message of the last failing call on this thread ("" if none).  The string
 * stays valid until the next call on the same thread. */
const char* cc_last_error(void);

/* Static text for a CC_* code. */
const char* cc_strerror(int code);

/* Compute units (num_cus) and XCDs (num_xcds) of HIP device `device`. */
int cc_device_query(int device, int32_t* num_cus, int32_t* num_xcds);

/* Bytes of the plan blob cc_plan would write for these inputs.
 * seqlens: host int32[batch]. */
int cc_plan_size(const cc_problem* prob, const cc_plan_opts* opts, const int32_t* seqlens,
                 size_t* bytes);

/* Build the work plan on the host (pure, deterministic, thread-safe).
 * seqlens: host int32[batch].  block_table: host int32[batch][max_pages_per_seq]
 * or NULL; when given, every page a sequence uses is checked to lie in
 * [0, num_pages) (CC_ERR_PAGE otherwise).  plan: host buffer of `bytes` bytes
 * (>= cc_plan_size).  The blob is self-describing (header + arrays, int32
 * little-endian); copy it verbatim to device memory for cc_decode.  Its header
 * holds a 32-bit FNV-1a hash of the problem's int32 fields (mode .. topk, in
 * struct order) followed by seqlens[0 .. batch), which cc_plan_check compares:
 * a plan serves only the lengths it was built for (GLM-5.2 decode article,
 * MegaRTP design: the host plan is rebuilt when the lengths change).        */
int cc_plan(const cc_problem* prob, const cc_plan_opts* opts, const int32_t* seqlens,
            const int32_t* block_table, void* plan, size_t bytes);

/* Shared-prefix decode (MeldKernel summary, "Experiments and results": the
 * shared-prefix experiment of Fig. 11).  Sequences b with prefix_group[b] = g
 * (-1: none; g < num_groups) begin with the same prefix_len[g] tokens, held in
 * the same pages of every member's block-table row.  The plan reads such a
 * prefix once per KV head for up to 16 / G members at a time (a "prefix
 * unit" whose 16 query rows are the members' G heads) and each sequence's own
 * KV only past its prefix; a prefix piece is one more split of each member,
 * merged by the same in-kernel log-sum-exp merge, so the result is the same
 * attention over each sequence's whole KV.
 *  - GQA with one query token; Hq / Hkv must divide 16; heads_per_unit = G;
 *    policy CC_POLICY_STREAMK (unit_cost as for cc_plan).
 *  - prefix_len[g]: a whole number of pages (0: the group shares nothing);
 *    every member's seqlens[b] >= prefix_len[g].
 *  - block_table (host, or NULL): when given, pages are checked as for
 *    cc_plan and every member of a group must name the same first
 *    prefix_len[g] / page_size pages (CC_ERR_INVALID otherwise).
 * The blob is used with cc_decode like any plan (the problem is unchanged).
 * cc_plan_check covers the lengths, not the grouping.                      */
int cc_plan_prefix_size(const cc_problem* prob, const cc_plan_opts* opts, const int32_t* seqlens,
                        const int32_t* prefix_group, int32_t num_groups, const int32_t* prefix_len,
                        size_t* bytes);
int cc_plan_prefix(const cc_problem* prob, const cc_plan_opts* opts, const int32_t* seqlens,
                   const int32_t* block_table, const int32_t* prefix_group, int32_t num_groups,
                   const int32_t* prefix_len, void* plan, size_t bytes);

/* ---------------------------------------------------- MoE grouped GEMM
 * The second imbalanced workload the method is instantiated on (MeldKernel
 * summary, "Problem and motivation": expert token counts differ from SM to
 * SM; "Core method": the mapping follows the real counts at run time).
 * Routed rows sorted by expert, expert e owning rows offsets[e] ..
 * offsets[e+1] - 1 (offsets = exclusive prefix sum of expert_tokens):
 *   Y[r, :] = X[r, :] . W[e]^T      (bf16 inputs, fp32 accumulation and out)
 *   x  bf16 [R][hidden], w bf16 [num_experts][out_dim][hidden] (row n of
 *   expert e is its output column n), y fp32 [R][out_dim], R = sum of
 *   expert_tokens.
 * The plan cuts the output into tiles of opts.heads_per_unit rows x 256
 * columns (unit = expert, column block, row block) and each tile's hidden
 * range into k tiles of opts.tile_tokens; the (tile, k tile) work is split
 * into num_cus equal chunks as for decode (CC_POLICY_STREAMK, unit_cost) or
 * one worker per output tile (CC_POLICY_PER_UNIT).  A tile split across
 * compute units is summed in split order by its last piece to finish
 * (cc_moe_gemm) or by a second kernel (cc_moe_gemm_variant with
 * CC_REDUCE_SPLIT_COMBINE).  cc_moe_gemm needs heads_per_unit = 256,
 * tile_tokens = 64, hidden % 64 == 0, out_dim % 256 == 0.  The plan blob has
 * the layout of a decode plan (mode CC_MODE_MOE) and works with
 * cc_workspace_size / cc_workspace_init / cc_workspace_check. */
typedef struct cc_moe_problem {
  int32_t num_experts;
  int32_t hidden;   /* K */
  int32_t out_dim;  /* N */
} cc_moe_problem;

/* Plan size / plan for these per-expert row counts (host int32[num_experts]). */
int cc_moe_plan_size(const cc_moe_problem* prob, const cc_plan_opts* opts, const int32_t* expert_tokens,
                     size_t* bytes);
int cc_moe_plan(const cc_moe_problem* prob, const cc_plan_opts* opts, const int32_t* expert_tokens, void* plan,
                size_t bytes);

/* Y for all experts in one persistent launch (device x, w, y, workspace;
 * host and device copies of the plan).  Asynchronous on `stream`. */
int cc_moe_gemm(const cc_moe_problem* prob, const void* plan_host, const void* plan_dev, const void* x,
                const void* w, float* y, void* workspace, size_t workspace_bytes, void* stream);

/* cc_moe_gemm with an explicit reduction of split tiles (CC_REDUCE_*). */
int cc_moe_gemm_variant(int reduce, const cc_moe_problem* prob, const void* plan_host, const void* plan_dev,
                        const void* x, const void* w, float* y, void* workspace, size_t workspace_bytes,
                        void* stream);

/* CC_OK if the host blob `plan` is a well-formed plan built for exactly `prob`
 * and these lengths (seqlens: host int32[batch]), else CC_ERR_PLAN with the
 * reason in cc_last_error().  Host only; no device work.  cc_decode cannot
 * make this check itself (its seqlens live in device memory); its kernels
 * instead flag a plan whose pieces do not end at seqlens (see cc_decode). */
int cc_plan_check(const void* plan, const cc_problem* prob, const int32_t* seqlens);

/* Device workspace bytes a plan needs: an error word, an arrival counter and
 * a merge-claim mask per unit, and one partial (m, l, o) slot per piece of a
 * split unit. */
int cc_workspace_size(const void* plan_host, size_t* bytes);

/* Zero a workspace (device, `bytes` long) on `stream` with a fill kernel.
 * Needed after allocation and whenever the plan used with the workspace
 * changes: every cc_decode leaves its plan's counters at zero, so calls with
 * one plan ordered on one stream can share a workspace, but another plan may
 * place its counters where the previous one kept partials.  Calls that may
 * run concurrently need separate workspaces. */
int cc_workspace_init(void* workspace, size_t bytes, void* stream);

/* Synchronous debug check of a workspace after the work on `stream`:
 * *dirty_counters = number of non-zero arrival counters and claim masks, *device_flags = the
 * device error word (bit 0: a plan item ran past seqlens[b]; bit 1: a page id
 * outside [0, num_pages); bit 2: a sparse index outside [0, seqlens[b])).
 * Returns CC_ERR_DEVICE_DATA if either is non-zero. */
int cc_workspace_check(const void* plan_host, const void* workspace, void* stream,
                       int32_t* dirty_counters, int32_t* device_flags);

/* Decode attention with the in-kernel just-in-time merge.
 * plan_host: the blob from cc_plan (host); plan_dev: the same bytes in device
 * memory.  q, k_cache, v_cache (NULL for MLA modes), block_table, seqlens,
 * indices (MLA_SPARSE, else NULL): device, layouts as in cc_problem.
 * out, lse: device outputs.  q, k_cache, v_cache, out and the workspace must
 * be 16-byte aligned (CC_ERR_INVALID otherwise; every torch allocation is).
 * workspace: device, >= cc_workspace_size bytes,
 * initialised once with cc_workspace_init.  Asynchronous on `stream`.  When
 * the plan holds empty sequences, a first small kernel writes their out (0)
 * and lse (-inf).
 * Host-side checks (before any launch): null pointers, plan header vs `prob`,
 * the plan's own structure (every item's unit, token range and split index
 * in range, worker offsets ascending), supported shapes, workspace size.
 * Device data is not validated on the host.  On the device:
 *  - a plan that does not match seqlens (a piece ends past seqlens[b], or the
 *    last piece of a unit ends before it) sets bit 0 of the workspace error
 *    word and turns that unit's out and lse into NaN: a stale plan never
 *    yields a plausible-looking result;
 *  - out-of-range page ids (bit 1) and sparse indices (bit 2) are clamped so
 *    no access leaves its buffer; the affected outputs are unspecified.
 * cc_workspace_check reports the error word. */
int cc_decode(const cc_problem* prob, const void* plan_host, const void* plan_dev, const void* q,
              const void* k_cache, const void* v_cache, const int32_t* block_table,
              const int32_t* seqlens, const int32_t* indices, float* out, float* lse,
              void* workspace, size_t workspace_bytes, void* stream);

/* cc_decode with an explicit reduction (CC_REDUCE_*): CC_REDUCE_FUSED is
 * cc_decode; CC_REDUCE_SPLIT_COMBINE writes all partials to the workspace and
 * merges them in a second kernel.  With a CC_POLICY_PER_UNIT plan nothing is
 * split and both reductions are the per-(sequence, head) launch. */
int cc_decode_variant(int reduce, const cc_problem* prob, const void* plan_host,
                      const void* plan_dev, const void* q, const void* k_cache,
                      const void* v_cache, const int32_t* block_table, const int32_t* seqlens,
                      const int32_t* indices, float* out, float* lse, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Bytes of the scratch array cc_decode_noalloc uses on each device (64 MiB:
 * the workspace of a 256-chunk plan for any of the five benchmark workloads,
 * up to 40 MiB for 64 DeepSeek-style MLA sequences of up to 16K tokens), and
 * the most units (query-head groups sharing one K/V stream) a plan may have
 * there: its first 2 MiB hold that many arrival counters at fixed places, so
 * the partials of one call never land on the counters of the next. */
#define CC_NOALLOC_WORKSPACE_BYTES (64u << 20)
#define CC_NOALLOC_MAX_UNITS 16384

/* cc_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  The
 * arguments are cc_decode's without the workspace: its partials, counters and
 * error word live instead in a library-owned device array of
 * CC_NOALLOC_WORKSPACE_BYTES, one per GPU, held until the process ends.
 *  - A plan with more than CC_NOALLOC_MAX_UNITS units, or whose partials do
 *    not fit beside the counters, returns CC_ERR_BUFFER before any device
 *    work; other errors as for cc_decode.
 *  - The call allocates nothing: no hipMalloc or hipFree, no allocating
 *    library routine.  The first call on a device looks up the array's address
 *    and enqueues one clear of it on `stream`.
 *  - Every call on a device shares that device's array, which keeps the last
 *    call's contents; calls with different plans may follow each other (the
 *    counters sit at fixed places and the kernels leave them at zero).  Calls
 *    on one device must be ordered (one stream, or streams ordered by
 *    events): overlapping calls race.
 *  - The device error word is not readable through this interface; a plan
 *    that does not match seqlens still turns the affected outputs into NaN. */
int cc_decode_noalloc(const cc_problem* prob, const void* plan_host, const void* plan_dev, const void* q,
                      const void* k_cache, const void* v_cache, const int32_t* block_table,
                      const int32_t* seqlens, const int32_t* indices, float* out, float* lse, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* CROSSCU_H */
