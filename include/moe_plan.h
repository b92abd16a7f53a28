/*
 * moe_plan -- expert-parallel dispatch planning for one MoE layer on MI355X.
 *
 * C ABI of the HIP library load_balance_planning_amd/libmoe_plan.so.
 *
 * The path turns a layer's gate logits into an expert-parallel dispatch plan:
 *   moe_plan_route     top-k gating + load histograms
 *   moe_plan_hist      the histograms alone, from a given top-k
 *   moe_plan_plan      hot-expert replication + token re-routing
 *   moe_plan_dispatch  dispatch layout + bf16 row gather
 *   moe_plan_step      route, plan and dispatch in one call
 *   moe_plan_combine   the return path: gate-weighted sum of expert outputs
 *   moe_plan_place     correlated expert placement from the co-selection counts
 *   moe_plan_dedup_count / moe_plan_dedup_dispatch
 *                      rows of a deduplicating dispatcher: counts, and the
 *                      layout with its bf16 row gather
 *   moe_plan_quality   plan-quality counters: rank-load imbalance, assignments
 *                      crossing nodes, assignments served by replicas
 *   moe_plan_predict   token-shuffle prediction: the rank expected to hold most
 *                      of each token's next-layer experts
 *   moe_plan_slot_map / moe_plan_replica_pull / moe_plan_replica_push
 *                      replica slots of a plan; expert parameters into the
 *                      slots, replica gradients back to the main ranks
 * EP ranks and NVLink domains ("nodes") are logical partitions on one GPU:
 *   source rank of token t   src(t)  = t / (T/R)     (contiguous token blocks)
 *   domain of rank r          dom(r)  = r / G         (contiguous rank blocks)
 *   main rank of expert e     main(e) = e / (E/R)     (contiguous expert blocks)
 *
 * Sources:
 *   [TopoEP]   "TopoEP: Topology-Aware Load Balancing for Expert-Parallel MoE
 *              Training": routing matrix (section 4.1, Eq. 3), domain demand
 *              (Eq. 4), constraints C1-C5 (section 4.2), two-stage solver
 *              (section 4.3, Eqs. 9 and 10, Fig. 9), device-resident plan that
 *              drives dispatch (sections 3.1 and 5).
 *   [Coupling] "Expert Coupling in MoE Pretraining": within-layer expert
 *              co-selection counts, layer-to-layer routing counts, correlated
 *              expert placement and deduplicated dispatch ("Moving Correlated
 *              Experts Together", Fig. 3).
 *
 * Conventions for every call
 *   - Pointers named in the structs are HIP device pointers unless stated.
 *     The caller allocates and owns every input and output buffer; sizes are
 *     fixed by the configuration (moe_plan_query reports them).  Layouts are
 *     dense row-major int32 / float32 / uint16 (bf16 bit patterns).
 *   - `stream` is a hipStream_t (NULL = the default stream).  The compute
 *     calls only enqueue work: they never allocate, never synchronise and
 *     never copy to the host.  One handle serves one stream at a time; calls
 *     on one stream run in order; every output is complete in `stream` order
 *     when the call's work ends.
 *   - A handle belongs to the HIP device that was current at moe_plan_create;
 *     each call runs on that device and gives the caller's current device
 *     back before it returns.  `stream` must belong to the handle's device.
 *   - Argument and configuration errors return a negative code synchronously
 *     and enqueue nothing.  A data-dependent error (a NaN gate logit) sets a
 *     device status word that moe_plan_status reads.
 *   - Every output is fully overwritten on each call; unused entries of the
 *     instance arrays are -1.  Results are deterministic: the same inputs give
 *     the same bytes on every run.
 */
#ifndef MOE_PLAN_H
#define MOE_PLAN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null pointer, bad size or inconsistent configuration */
  MOE_ERR_UNSUPPORTED = -2, /* valid but beyond the library's limits (see moe_plan_create) */
  MOE_ERR_HIP = -3,         /* a HIP runtime call failed */
  MOE_ERR_NONFINITE = -4,   /* status flag: a gate logit was NaN */
  MOE_ERR_INTERNAL = -5     /* status flag: an internal consistency check failed on the device */
};

/* Status-word bits reported by moe_plan_status. */
#define MOE_STATUS_NAN_LOGIT 1
#define MOE_STATUS_PLAN_CHECK 2
#define MOE_STATUS_BAD_TOPK 4   /* a top-k entry out of [0, E) or repeated within a token */
#define MOE_STATUS_BAD_PAIRS 8  /* moe_plan_place: a co-selection count < 0, a non-zero diagonal
                                   entry or a row sum >= 2^31 */
#define MOE_STATUS_BAD_KEY 16   /* moe_plan_dedup_*: a slot key outside the table, or a table
                                   entry outside [0, R) */
#define MOE_STATUS_BAD_OMEGA 32 /* moe_plan_plan: the routing matrix is not the one of the top-k
                                   it was given with */

typedef struct moe_plan* moe_plan_t;

/*
 * Layer configuration.
 *   T  tokens of all ranks (multiple of R; 0 allowed)
 *   E  routed experts (multiple of R);  k  top-k (1 <= k <= E)
 *   R  logical EP ranks;  G  ranks per NVLink domain (R multiple of G), M = R/G domains
 *   H  hidden size in bf16 elements per token row
 *   replica_budget  B: extra expert instances per layer over all ranks; domain d
 *                   may add B_d = B/M (+1 for d < B mod M)
 *   slots_per_rank  N_slot replica slots per rank [TopoEP C3]; <= 0 derives
 *                   ceil(ceil(B/M)/G)
 *   expert_bytes    ||W_e|| in bytes; < 0 derives 9*H*H/4 (three H x 3H/8 bf16
 *                   matrices: 9 MiB at H = 2048, the [TopoEP] Fig. 3 example)
 *   token_bytes     S_tok in bytes; <= 0 derives 2*H (one bf16 row)
 *   max_refine_iters  cap on intra-node refinement iterations per domain;
 *                   <= 0 derives 4096
 */
typedef struct {
  int32_t T, E, k, R, G, H;
  int32_t replica_budget;
  int32_t slots_per_rank;
  int64_t expert_bytes;
  int64_t token_bytes;
  int32_t max_refine_iters;
} moe_plan_config;

/* Element counts of every caller-owned buffer for a configuration. */
typedef struct {
  int64_t topk;          /* T*k      topk_idx, topk_val, slot_inst, slot_rank, perm, slot_pos */
  int64_t omega;         /* R*E      omega */
  int64_t experts;       /* E        expert_count */
  int64_t pair;          /* E*E      cooc, trans */
  int64_t inst_cap;      /* E+B      inst_expert, inst_rank, inst_load */
  int64_t quota;         /* R*(E+B)  quota */
  int64_t inst_offset;   /* E+B+1 */
  int64_t rank_offset;   /* R+1 */
  int64_t dispatch_elems;/* T*k*H    bf16 elements of the dispatch buffer */
  int64_t n_slot;        /* derived N_slot */
  int64_t expert_bytes;  /* derived ||W_e|| */
  int64_t token_bytes;   /* derived S_tok */
  int64_t max_refine_iters;
  int64_t workspace_bytes; /* device memory the handle owns */
} moe_plan_sizes;

/*
 * Outputs of moe_plan_route / moe_plan_hist.
 *   topk_idx   int32 [T][k]: the k experts of each token, largest logit first;
 *              equal logits order by lower expert index; -0.0 equals +0.0.
 *   topk_val   float [T][k] (nullable): bit copy of the selected logits.
 *   expert_count int32 [E]: assignments per expert.
 *   omega      int32 [R][E]: routing matrix, assignments of source rank s that
 *              select expert e [TopoEP Eq. 3].
 *   cooc       int32 [E][E] (nullable): tokens selecting both a and b, a != b;
 *              zero diagonal [Coupling, within-layer co-selection].
 *   trans      int32 [E][E] (nullable; written only when prev_topk is given):
 *              tokens selecting a in the previous layer and b in this one
 *              [Coupling, cross-layer routing].
 */
typedef struct {
  int32_t* topk_idx;
  float* topk_val;
  int32_t* expert_count;
  int32_t* omega;
  int32_t* cooc;
  int32_t* trans;
} moe_route_out;

/*
 * Outputs of moe_plan_plan.
 *   n_inst       int32 [1]: number of expert instances (E + replicas).
 *   inst_expert, inst_rank, inst_load  int32 [E+B]: instance i is an instance
 *                of expert inst_expert[i] on rank inst_rank[i] executing
 *                inst_load[i] assignments (U[e][r]).  Instances are
 *                rank-major; on each rank its main experts (ascending) come
 *                first, then its replicas (ascending expert).  Entries from
 *                n_inst on are -1.
 *   rank_load    int32 [R]: L_r, assignments executed on rank r [TopoEP 4.2].
 *   quota        int32 [R][E+B]: q[s][i], assignments of source s run on
 *                instance i (zero for i >= n_inst).
 *   slot_inst    int32 [T*k]: instance of slot t*k+j.
 *   slot_rank    int32 [T*k]: the slot's position among the slots of its
 *                instance, in slot order (the stable rank the dispatch layout
 *                adds to the instance's first row).
 */
typedef struct {
  int32_t* n_inst;
  int32_t* inst_expert;
  int32_t* inst_rank;
  int32_t* inst_load;
  int32_t* rank_load;
  int32_t* quota;
  int32_t* slot_inst;
  int32_t* slot_rank;
} moe_plan_out;

/*
 * Outputs of moe_plan_dispatch.
 *   perm         int32 [T*k]: slot id (t*k+j) at each dispatch row.
 *   slot_pos     int32 [T*k]: dispatch row of each slot (inverse of perm).
 *   inst_offset  int32 [E+B+1]: first dispatch row of each instance (the
 *                exclusive prefix of the instance loads); entry n_inst is
 *                T*k, later entries are -1.  These are the receive counts of
 *                the dispatch, derived on the device [TopoEP section 5].
 *   rank_offset  int32 [R+1]: first dispatch row of each rank; entry R is T*k.
 *                Rank r's rows [rank_offset[r], rank_offset[r+1]) are what an
 *                all-to-all would send to rank r.
 *   dispatch     uint16 [T*k][H]: bf16 rows, dispatch[pos] = hidden[perm[pos]/k].
 */
typedef struct {
  int32_t* perm;
  int32_t* slot_pos;
  int32_t* inst_offset;
  int32_t* rank_offset;
  uint16_t* dispatch;
} moe_dispatch_out;

/*
 * Outputs of moe_plan_place.
 *   expert_rank   int32 [E]: rank holding expert e.
 *   rank_experts  int32 [R][E/R]: the experts of each rank, ascending.  Giving
 *                 expert rank_experts[p] the new id p turns the placement into
 *                 the contiguous one moe_plan_plan assumes (main(e) = e/(E/R)):
 *                 permute the router's expert columns accordingly.
 *   intra         int64 [1]: co-selection weight kept inside ranks, the sum
 *                 over expert pairs a < b on one rank of cooc[a][b].
 *   n_swaps       int32 [1]: refinement swaps applied.
 */
typedef struct {
  int32_t* expert_rank;
  int32_t* rank_experts;
  int64_t* intra;
  int32_t* n_swaps;
} moe_place_out;

/*
 * Outputs of moe_plan_dedup_count / moe_plan_dedup_dispatch.  Slot q = t*k+j
 * goes to destination rank key_rank[slot_key[q]]; token t comes from source
 * rank t / (T/R).
 *   tok_ranks        int32 [T]: distinct destination ranks of token t.
 *                    (With T = 0 the per-token and per-row pointers may be NULL.)
 *   rank_rows        int32 [R][R]: rows sent from source s to rank r with
 *                    deduplication -- tokens of s with at least one slot on r.
 *   rank_slots       int32 [R][R] (nullable): slots of source s on rank r (one
 *                    row each without deduplication).
 * moe_plan_dedup_dispatch only (ignored by moe_plan_dedup_count):
 *   n_rows           int32 [1]: rows of the deduplicated dispatch (sum of tok_ranks).
 *   row_token        int32 [T*k]: token of each row; rows are ordered by
 *                    destination rank, then token.  Entries from n_rows on are -1.
 *   row_slots        int32 [T*k]: bit j set when slot j of the row's token goes
 *                    to the row's rank (the local experts it serves); -1 past n_rows.
 *   rank_row_offset  int32 [R+1]: first row of each rank; entry R is n_rows.
 *   slot_row         int32 [T*k]: row carrying slot q.
 *   ddispatch        uint16 [T*k][H] bf16: row p = hidden[row_token[p]];
 *                    rows from n_rows on are not written.
 */
typedef struct {
  int32_t* tok_ranks;
  int32_t* rank_rows;
  int32_t* rank_slots;
  int32_t* n_rows;
  int32_t* row_token;
  int32_t* row_slots;
  int32_t* rank_row_offset;
  int32_t* slot_row;
  uint16_t* ddispatch;
} moe_dedup_out;

/*
 * Outputs of moe_plan_predict.
 *   pred         int32 [T]: predicted rank of each token (NULL allowed when T = 0).
 *   rank_tokens  int32 [R]: tokens predicted for each rank.
 *   local        int64 [2] (nullable): with the next layer's top-k, its slots
 *                on the predicted rank (local[0]) and on the token's own
 *                source rank t / (T/R) (local[1], no shuffling).
 */
typedef struct {
  int32_t* pred;
  int32_t* rank_tokens;
  int64_t* local;
} moe_predict_out;

/*
 * Outputs of moe_plan_slot_map (N_slot = moe_plan_sizes.n_slot).
 *   slot_expert  int32 [R][N_slot]: expert held by slot j of rank r, -1 empty.
 *   slot_main    int32 [R][N_slot]: its main rank e / (E/R), -1 empty -- the
 *                source of the parameters and destination of the gradients.
 *   inst_slot    int32 [E+B]: slot of each replica instance on its rank; -1
 *                for main instances and unused entries.
 */
typedef struct {
  int32_t* slot_expert;
  int32_t* slot_main;
  int32_t* inst_slot;
} moe_slot_out;

/* Buffer sizes for a configuration (host only, no GPU work).  Returns
 * MOE_ERR_INVALID_ARG / MOE_ERR_UNSUPPORTED as moe_plan_create would. */
int moe_plan_query(const moe_plan_config* cfg, moe_plan_sizes* sizes);

/*
 * Validate cfg, bind the current HIP device and allocate the handle's
 * workspace (it may synchronise).  Limits of the library: E <= 2048, k <= 32,
 * R <= 256, G <= 64, B <= 1024, E/R + N_slot <= 1024, T < 2^22, T*k < 2^31,
 * H >= 1.
 * On success *out is a new handle; on error *out is NULL.
 */
int moe_plan_create(const moe_plan_config* cfg, moe_plan_t* out);

/*
 * Top-k gating and histograms of one layer.  logits: float [T][E] (device).
 * prev_topk: int32 [T][k] of the previous layer (nullable); out->trans is
 * written only when both prev_topk and out->trans are non-null.  Required
 * outputs: topk_idx, expert_count, omega.  A NaN logit sets
 * MOE_STATUS_NAN_LOGIT (that token's outputs are then unspecified); a bad
 * prev_topk row (entry outside [0, E) or repeated) MOE_STATUS_BAD_TOPK.
 * Sources: [TopoEP] section 2.1 (top-k gating) and Eq. 3; [Coupling].
 */
int moe_plan_route(moe_plan_t h, const float* logits, const int32_t* prev_topk,
                   const moe_route_out* out, void* stream);

/*
 * The histogram half of moe_plan_route from a given top-k: topk_idx int32
 * [T][k] (device, each row k distinct experts in [0, E); otherwise
 * MOE_STATUS_BAD_TOPK is set and the histograms are unspecified).  Writes
 * expert_count, omega and the nullable cooc / trans of out; out->topk_idx
 * and out->topk_val are ignored.
 */
int moe_plan_hist(moe_plan_t h, const int32_t* topk_idx, const int32_t* prev_topk,
                  const moe_route_out* out, void* stream);

/*
 * Replica placement and token re-routing [TopoEP section 4.3].  As in the
 * page's design, the input is the routing matrix of all ranks plus the layer
 * configuration [TopoEP abstract and section 3.1]; the top-k that the matrix
 * counts is passed too, for the per-slot instances:
 *   omega     int32 [R][E] (device): omega[s][e], assignments of source s to
 *             expert e [TopoEP Eq. 3] -- e.g. moe_plan_route's omega, or the
 *             matrix gathered from every rank;
 *   topk_idx  int32 [T][k] (device): each row k distinct experts in [0, E);
 *             token t belongs to source t / (T/R).  (NULL allowed when T = 0.)
 * omega must be the routing matrix of topk_idx: a mismatch sets
 * MOE_STATUS_BAD_OMEGA, a bad top-k row MOE_STATUS_BAD_TOPK, and the outputs
 * are then unspecified (every index still stays inside its buffer).  The
 * plan itself:
 *   D[d][e] = sum of omega over the sources of domain d (Eq. 4);
 *   stage 1 (inter-node placement): per domain, experts whose main instance is
 *     elsewhere with benefit b = 2*D*S_tok - ||W_e|| > 0 (Eq. 9), in
 *     descending b (ties: lower e), each to the rank of the domain with the
 *     fewest replicas and a free slot (ties: lower rank), within B_d;
 *   stage-1 routing: each (s, e) demand to the instances of e in dom(s) if
 *     any, else to all instances of e, split evenly (floor; the remainder one
 *     each to the first instances in rank order);
 *   stage 2 (intra-node refinement, Eq. 10): per domain, repeatedly move
 *     delta = min(U[e][r_b], floor((L_b - L_t)/2)) >= 1 assignments from the
 *     busiest rank r_b (ties: lower rank) to a rank r_t of the domain that
 *     hosts e or has a free slot, choosing the largest delta, then the lowest
 *     L_t, then an existing instance before a new replica, then lower e,
 *     then lower r_t; at most max_refine_iters moves per domain;
 *   quotas: per expert, demands omega[s][e] are matched to the instance loads
 *     in three passes -- the source's own rank, its domain, anywhere -- each
 *     pass sources ascending, instances in rank order;
 *   slot instances: the p-th slot (token order) of source s and expert e goes
 *     to the first instance whose running quota sum exceeds p; slot_rank is
 *     its position among its instance's slots in slot order.
 */
int moe_plan_plan(moe_plan_t h, const int32_t* omega, const int32_t* topk_idx, const moe_plan_out* out,
                  void* stream);

/*
 * Dispatch layout and bf16 gather [TopoEP section 5: the plan stays on the
 * device and the receive counts are derived there].  The receive counts are
 * the instance loads: inst_offset is their exclusive prefix (instances are
 * rank-major, so rank_offset follows), and the slots are laid out as a stable
 * counting sort by instance: slot_pos = inst_offset[slot_inst] + slot_rank.
 * hidden: uint16 [T][H] bf16 rows (device).  Reads plan->n_inst, inst_rank,
 * inst_load, slot_inst and slot_rank.  A plan whose positions fall outside
 * [0, T*k) sets MOE_STATUS_PLAN_CHECK and those slots are not copied.
 */
int moe_plan_dispatch(moe_plan_t h, const moe_plan_out* plan, const uint16_t* hidden,
                      const moe_dispatch_out* out, void* stream);

/*
 * One whole pass of the path in a single call: moe_plan_route, then
 * moe_plan_plan on its omega and topk_idx, then moe_plan_dispatch -- the
 * same outputs, bit for bit, as the three calls in order.  Inside the call
 * the routing-matrix output and the pair counts (route->cooc,
 * route->trans) are computed by extra workgroups of the solver launch, on the
 * CUs the single solver workgroup leaves idle (the pair counts' partial sums
 * are added by extra workgroups of the quota launch), so every kernel of the
 * call runs on `stream`.  The call keeps no state in the handle from one
 * call to the next (its routing-matrix accumulator is zero again when the
 * call's work ends), so it can be captured into a HIP graph and the graph
 * replayed, with the same pointers, in place of the call.  Sources: those of
 * the three calls.
 */
int moe_plan_step(moe_plan_t h, const float* logits, const int32_t* prev_topk, const uint16_t* hidden,
                  const moe_route_out* route, const moe_plan_out* plan, const moe_dispatch_out* out,
                  void* stream);

/*
 * moe_plan_step without a handle and without any allocation, for callers that
 * cannot call hipMalloc: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  It runs the launches of moe_plan_step
 * (same outputs, bit for bit) on the current HIP device, with the workspace in
 * a fixed 32 MiB device array of the library (one per GPU, held until the
 * process ends; the DeepSeek-V3-shaped layer with co-selection counts needs
 * about 11 MiB).  A configuration whose workspace does not fit returns
 * MOE_ERR_UNSUPPORTED and enqueues nothing; configuration and argument errors
 * return as from moe_plan_create / moe_plan_step.
 *   status  int32 [1] (device, caller-owned): zeroed by the call, then the
 *           MOE_STATUS_* bits of this call (there is no moe_plan_status here).
 * Every call on one GPU shares that GPU's array: calls that overlap in time on
 * one GPU (other streams, other threads) race and give unspecified results.
 * Calls on one stream are ordered and safe.
 */
int moe_plan_step_static(const moe_plan_config* cfg, const float* logits, const int32_t* prev_topk,
                         const uint16_t* hidden, const moe_route_out* route, const moe_plan_out* plan,
                         const moe_dispatch_out* out, int32_t* status, void* stream);

/*
 * Gate-weighted combine, the return path of the dispatch [TopoEP section 2.1,
 * Fig. 1]: for every token t,
 *   out[t][:] = bf16( sum over j = 0..k-1 of w[t][j] * expert_out[slot_pos[t*k+j]][:] )
 * with w[t][*] the softmax of the k selected logits topk_val[t][*] (their
 * maximum subtracted before exp), accumulated in fp32 in slot order and
 * rounded once to bf16, nearest even.  The weights are a reading: the pages
 * do not define them.
 *   topk_val    float [T][k] (device): moe_plan_route's topk_val.
 *   slot_pos    int32 [T*k] (device): moe_plan_dispatch's slot_pos.
 *   expert_out  uint16 [T*k][H] bf16 rows in dispatch order (device).
 *   out         uint16 [T][H] bf16 (device), fully overwritten.
 * A non-finite selected logit sets MOE_STATUS_NAN_LOGIT (that token's output
 * is then unspecified); a position outside [0, T*k) sets
 * MOE_STATUS_PLAN_CHECK and the slot is skipped.
 */
int moe_plan_combine(moe_plan_t h, const float* topk_val, const int32_t* slot_pos, const uint16_t* expert_out,
                     uint16_t* out, void* stream);

/*
 * Correlated expert placement [Coupling, "Moving Correlated Experts
 * Together"]: the experts are partitioned over the R ranks, exactly E/R per
 * rank, so that frequently co-selected experts share a rank.  The page gives
 * the goal and the fixed count per rank, not an algorithm; this one maximises
 * intra (see moe_place_out) by greedy growth then pair-swap refinement:
 *   growth      ranks 0..R-1 in order; the first expert of a rank is the
 *               unplaced one with the largest sum_x cooc[e][x], each further
 *               one the unplaced expert with the largest co-selection with the
 *               rank's experts so far; ties to the lower expert id;
 *   refinement  swap the experts a < b (on different ranks) whose exchange
 *               raises intra the most (ties: lower a, then lower b) while the
 *               gain is positive, at most max_swaps times (< 0: 4096).
 * cooc: int32 [E][E] (device) as moe_plan_route writes it -- symmetric, zero
 * diagonal, entries >= 0, row sums < 2^31.  A negative entry, a non-zero
 * diagonal or a row sum >= 2^31 sets MOE_STATUS_BAD_PAIRS (the result is
 * then a valid partition but otherwise unspecified); asymmetric input is not
 * detected and gives an unspecified partition.  Four launches: the passes
 * over all of cooc run on the whole chip, the growth and the refinement in
 * one workgroup each; time grows with E (a sequential greedy step per
 * expert).  Uses the handle's workspace, so calls on one handle run in
 * stream order.
 */
int moe_plan_place(moe_plan_t h, const int32_t* cooc, int32_t max_swaps, const moe_place_out* out,
                   void* stream);

/*
 * Deduplicated row counts [Coupling, "Moving Correlated Experts Together",
 * Fig. 3: a token sends one row to each destination rank, however many of its
 * experts live there].  slot_key int32 [T*k] (device): top-k expert ids or
 * instance ids.  key_rank int32 [n_keys] (device, nullable): rank of each key
 * -- a placement's expert_rank, or moe_plan_plan's inst_rank (n_keys = E+B);
 * NULL means the contiguous placement key / (E/R) with keys in [0, E).  A key
 * outside the table, or a table entry outside [0, R), sets MOE_STATUS_BAD_KEY
 * and that slot is left out.  Writes tok_ranks, rank_rows and, when non-null,
 * rank_slots.
 */
int moe_plan_dedup_count(moe_plan_t h, const int32_t* slot_key, const int32_t* key_rank, int32_t n_keys,
                         const moe_dedup_out* out, void* stream);

/*
 * Deduplicated dispatch: the counts of moe_plan_dedup_count, the row layout
 * (rank-major, tokens ascending within a rank: row of (r, t) = rank_row_offset[r]
 * + number of earlier tokens with a slot on r) and the bf16 row copy --
 * each hidden row read once and written to its token's distinct ranks.
 * hidden: uint16 [T][H] (device).  A left-out slot (bad key) has slot_row -1.
 */
int moe_plan_dedup_dispatch(moe_plan_t h, const int32_t* slot_key, const int32_t* key_rank, int32_t n_keys,
                            const uint16_t* hidden, const moe_dedup_out* out, void* stream);

/*
 * Plan-quality counters [TopoEP section 6.2 Fig. 10 and section 6.4 Fig. 13(b):
 * rank-load imbalance = largest rank load / mean; section 6.6 Fig. 16: the
 * shares of assignments executed on another node than their source and
 * executed by replicas].  From moe_plan_plan's n_inst, inst_expert,
 * inst_rank, rank_load and quota (device), writes int64 out[8] (device):
 *   out[0] assignments (sum of the quotas)     out[1] on the source's own rank
 *   out[2] on the source's node                out[3] on another node
 *   out[4] on a replica (rank != e / (E/R))     out[5] largest rank load
 *   out[6] smallest rank load                  out[7] replicas (n_inst - E)
 * The imbalance is out[5] * R / out[0].  An n_inst outside [E, E+B] or an
 * instance with a rank or expert out of range sets MOE_STATUS_PLAN_CHECK.
 */
int moe_plan_quality(moe_plan_t h, const moe_plan_out* plan, int64_t* out, void* stream);

/*
 * Token-shuffle prediction [Coupling, "Moving Tokens Toward Their Next
 * Experts": a token's experts at this layer predict the GPU holding most of its
 * next-layer experts, and the token moves there before the next router].  The
 * page gives no formula; each of the token's experts a votes with its
 * empirical next-layer distribution over ranks:
 *   P[a][r]  = (sum over experts b on rank r of trans[a][b]) / count_cur[a]
 *              (0 when count_cur[a] = 0)
 *   score[r] = P[a_0][r] + ... + P[a_{k-1}][r]   (IEEE double, slot order)
 *   pred[t]  = argmax_r score[r], ties to the lower rank.
 * topk_cur   int32 [T][k] this layer's top-k (device).
 * trans      int32 [E][E] transitions from this layer to the next (device):
 *            moe_plan_route's trans of the next layer (its prev_topk = topk_cur),
 *            or counts gathered earlier.
 * count_cur  int32 [E] this layer's expert counts (device).
 * key_rank   int32 [E] (device, nullable): rank of each next-layer expert;
 *            NULL means the contiguous placement b / (E/R).
 * topk_next  int32 [T][k] (device, nullable): the next layer's top-k, for
 *            out->local.
 * An expert id out of range sets MOE_STATUS_BAD_TOPK (that slot is left out),
 * a rank out of range MOE_STATUS_BAD_KEY, a negative count
 * MOE_STATUS_BAD_PAIRS.
 */
int moe_plan_predict(moe_plan_t h, const int32_t* topk_cur, const int32_t* trans, const int32_t* count_cur,
                     const int32_t* key_rank, const int32_t* topk_next, const moe_predict_out* out, void* stream);

/*
 * Replica slots [TopoEP section 3.2, Replica Buffer Management, and Fig. 6:
 * every rank keeps N_slot preallocated replica slots; the plan's mapping from
 * occupied slots to experts names the main rank that supplies a replica's
 * BF16 parameters in the forward pass and receives its gradients in the
 * backward pass].  The replicas of rank r fill its slots in instance order
 * (ascending expert); the rest are empty.  Reads plan->n_inst, inst_expert,
 * inst_rank (device).  A plan whose instances are not rank-major with main
 * experts first, or with more replicas on a rank than N_slot, sets
 * MOE_STATUS_PLAN_CHECK.
 */
int moe_plan_slot_map(moe_plan_t h, const moe_plan_out* plan, const moe_slot_out* out, void* stream);

/*
 * Parameter pull into the replica slots: replica_params[r][j][:] =
 * main_params[slot_expert[r][j]][:] for every occupied slot, param_elems bf16
 * elements per expert.  main_params: uint16 [E][param_elems] (rank m owns rows
 * m*E/R ... (m+1)*E/R-1); replica_params: uint16 [R][N_slot][param_elems]
 * (device); empty slots are not written.
 */
int moe_plan_replica_pull(moe_plan_t h, const int32_t* slot_expert, const uint16_t* main_params,
                          int64_t param_elems, uint16_t* replica_params, void* stream);

/*
 * Gradient return from the replica slots: for the expert e in slot j of rank
 * r and m = e / (E/R), grad_accum[m][r][e - m*E/R][:] = replica_grads[r][j][:]
 * -- main rank m's gradient buffer, split by source rank.  replica_grads:
 * uint16 [R][N_slot][param_elems]; grad_accum: uint16 [R][R][E/R][param_elems]
 * (device); regions of no slot are not written.
 */
int moe_plan_replica_push(moe_plan_t h, const int32_t* slot_expert, const uint16_t* replica_grads,
                          int64_t param_elems, uint16_t* grad_accum, void* stream);

/*
 * Kernel timing for roofline reports [the measurement the pages' own solver
 * latencies come from: HIP events, TopoEP section 6.3].  gather_begin and
 * gather_end are hipEvent_t handles (created by the caller, on the handle's
 * device) or both NULL to stop.  While set, every moe_plan_dispatch and
 * moe_plan_step of this handle records gather_begin on its stream right
 * before the launch of its row copy (the gather kernel) and gather_end right
 * after it, so that hipEventElapsedTime gives that one kernel's duration.
 * Host call; enqueues nothing.
 */
int moe_plan_set_events(moe_plan_t h, void* gather_begin, void* gather_end);

/*
 * Orders the row copies of handles that pipeline batches on separate streams
 * [TopoEP section 3.3: chunks of a step overlap one another's communication
 * and computation].  wait_event and done_event are hipEvent_t handles of the
 * handle's device (each nullable).  While set, every moe_plan_dispatch and
 * moe_plan_step of this handle makes its stream wait for wait_event (its most
 * recent record when the call is made) right before the launch of its row
 * copy, and records done_event right after it.  Chaining two handles A and B
 * (A waits for B's done event and B for A's) runs their copies one after the
 * other at full bandwidth while each batch's top-k, plan and quotas run beside
 * the other batch's copy; without it the two copies tend to run at the same
 * time, at half the bandwidth each, and the small kernels of both batches
 * then run with nothing to hide behind.  While either event is set, the
 * handle's solver launch is also sized to be placed beside the other
 * handle's running copy (256-thread workgroups within the LDS that copy
 * leaves free) instead of for running alone (512-thread workgroups); the
 * outputs are the same either way.  Host call; enqueues nothing.
 */
int moe_plan_set_gather_order(moe_plan_t h, void* wait_event, void* done_event);

/*
 * Figures of a HIP device for roofline reports (host call, no handle):
 * out[0] compute units, out[1] peak shader clock (kHz), out[2] peak memory
 * clock (kHz), out[3] memory bus width (bits), out[4] L2 cache bytes,
 * out[5] device memory bytes.
 */
int moe_plan_device_info(int device, int64_t* out);

/*
 * Wait for the work of the handle's last call (it synchronises that call's
 * stream only, which must still exist), copy the device status word to
 * *host_flags (MOE_STATUS_* bits, 0 when clean) and clear it.  Not for use
 * while that stream is being captured into a graph.
 */
int moe_plan_status(moe_plan_t h, int32_t* host_flags);

/* Free the handle's workspace (synchronises the device).  NULL is a no-op. */
void moe_plan_destroy(moe_plan_t h);

#ifdef __cplusplus
}
#endif
#endif /* MOE_PLAN_H */
