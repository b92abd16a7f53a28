/*
 * CPU oracle for the MoE dispatch-planning path -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, single-threaded C++ implementation of what the path
 * computes, used to check the HIP library output byte for byte.  Only the
 * tests, the smoke check and the benchmark's CPU-baseline leg may load it;
 * the product path never calls it and shares no code with it.
 *
 * Sources (cited by page title and section / equation):
 *   [TopoEP]  "TopoEP: Topology-Aware Load Balancing for Expert-Parallel MoE
 *             Training" -- routing matrix (Eq. 3), domain demand (Eq. 4),
 *             constraints C1-C5 (section 4.2), two-stage solver (section 4.3,
 *             Eqs. 9 and 10, Fig. 9).
 *   [Coupling] "Expert Coupling in MoE Pretraining" -- within-layer expert
 *             co-selection counts and layer-to-layer routing counts.
 *   Combine: [TopoEP] section 2.1, Fig. 1 (the return path of the dispatch);
 *             the gate weights are a reading (softmax of the selected logits).
 *   Placement and deduplication: [Coupling] "Moving Correlated Experts
 *             Together", Fig. 3 (the partition algorithm is a reading).
 *   Plan quality: [TopoEP] sections 6.2, 6.4, 6.6 (Figs. 10, 13(b), 16).
 *   Token-shuffle prediction: [Coupling] "Moving Tokens Toward Their Next
 *             Experts" (the scoring rule is a reading).
 *   Replica slots and transfers: [TopoEP] section 3.2, Fig. 6.
 *
 * Every function returns 0 on success or a negative status:
 *   -1 invalid argument / configuration, -4 a NaN gate logit,
 *   -5 an internal consistency check failed.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t T;          /* tokens of all ranks, contiguous blocks of T/R per source rank */
  int32_t E;          /* routed experts; main(e) = e / (E/R) */
  int32_t k;          /* top-k */
  int32_t R;          /* EP ranks */
  int32_t G;          /* ranks per NVLink domain; dom(r) = r / G */
  int32_t H;          /* hidden size (bf16 elements per token row) */
  int32_t B;          /* replica budget: extra instances per layer, all domains together */
  int32_t n_slot;     /* replica slots per rank; <= 0 derives ceil(ceil(B/M)/G) */
  int64_t W;          /* expert parameter bytes; < 0 derives 9*H*H/4 */
  int64_t S;          /* bytes of one routed activation; <= 0 derives 2*H */
  int32_t max_iters;  /* intra-node refinement iterations per domain; <= 0 derives 4096 */
} oracle_cfg;

/* Derived parameters: out[0..7] = M, T_r, E_r, n_slot, S, W, max_iters, B (as given). */
int oracle_params(const oracle_cfg* c, int64_t* out);
/* Per-domain replica budget B_d for d in [0, M). */
int oracle_domain_budget(const oracle_cfg* c, int32_t* out_bd);

/* Top-k selection plus histograms.  prev_topk / trans and cooc may be NULL. */
int oracle_route(const oracle_cfg* c, const float* logits, const int32_t* prev_topk,
                 int32_t* topk_idx, float* topk_val, int32_t* count, int32_t* omega,
                 int32_t* cooc, int32_t* trans);

/* Two-stage replica placement, token routing, quotas and per-slot instances.
 * rank_load_stage1 (R entries), trace (trace_cap records of 7 int32) and
 * n_trace may be NULL.  A trace record is
 * {domain, iteration, r_busy, expert, r_target, delta, created_replica}. */
int oracle_plan(const oracle_cfg* c, const int32_t* omega, const int32_t* topk_idx,
                int32_t* n_inst, int32_t* inst_expert, int32_t* inst_rank, int32_t* inst_load,
                int32_t* rank_load, int32_t* quota, int32_t* slot_inst,
                int32_t* rank_load_stage1, int32_t* trace, int32_t trace_cap, int32_t* n_trace);

/* Stable counting-sort layout of the slots by instance, then the row copy.
 * slot_rank (T*k) receives each slot's position inside its instance segment.
 * dispatch may be NULL (layout only). */
int oracle_dispatch(const oracle_cfg* c, int32_t n_inst, const int32_t* inst_rank,
                    const int32_t* slot_inst, const uint16_t* hidden,
                    int32_t* perm, int32_t* slot_pos, int32_t* inst_offset, int32_t* rank_offset,
                    int32_t* slot_rank, uint16_t* dispatch);

/* Gate-weighted combine, in double: out[t][h] = sum_j w[t][j] *
 * expert_out[slot_pos[t*k+j]][h] with w the softmax of the k selected logits
 * topk_val[t][*].  expert_out: bf16 rows [T*k][H] in dispatch order. */
int oracle_combine(const oracle_cfg* c, const float* topk_val, const int32_t* slot_pos,
                   const uint16_t* expert_out, double* out);

/* Correlated expert placement: partition of the E experts over the R ranks,
 * exactly E/R per rank, maximising the co-selection weight kept inside ranks
 * (greedy growth, then pair-swap refinement, at most max_swaps swaps;
 * max_swaps < 0 means 4096).  cooc: int32 [E][E] as oracle_route writes it.
 * expert_rank [E]; rank_experts [R][E/R] (ascending within a rank);
 * intra [1] the kept weight; n_swaps [1]. */
int oracle_place(const oracle_cfg* c, const int32_t* cooc, int32_t max_swaps, int32_t* expert_rank,
                 int32_t* rank_experts, int64_t* intra, int32_t* n_swaps);

/* Deduplicated row counts.  Slot q goes to rank key_rank[slot_key[q]]
 * (key_rank NULL: slot_key[q] / (E/R)).  tok_ranks [T]; rank_rows [R][R];
 * rank_slots [R][R] nullable. */
int oracle_dedup(const oracle_cfg* c, const int32_t* slot_key, const int32_t* key_rank, int32_t n_keys,
                 int32_t* tok_ranks, int32_t* rank_rows, int32_t* rank_slots);

/* Deduplicated dispatch layout (rows by rank, then token) and row copy.
 * Capacity T*k rows; k <= 32.  ddispatch nullable. */
int oracle_dedup_dispatch(const oracle_cfg* c, const int32_t* slot_key, const int32_t* key_rank,
                          int32_t n_keys, const uint16_t* hidden, int32_t* n_rows, int32_t* row_token,
                          int32_t* row_slots, int32_t* rank_row_offset, int32_t* slot_row,
                          uint16_t* ddispatch);

/* Plan quality [TopoEP Figs. 10, 13(b), 16]: out[8] = assignments, same rank,
 * same node, other node, served by replicas, largest and smallest rank
 * load, replicas. */
int oracle_quality(const oracle_cfg* c, int32_t n_inst, const int32_t* inst_expert, const int32_t* inst_rank,
                   const int32_t* rank_load, const int32_t* quota, int64_t* out);

/* Token-shuffle prediction [Coupling]: pred [T] = the rank with the largest
 * sum over the token's experts a of (transitions from a to that rank's
 * experts) / count_cur[a], in double, ties to the lower rank; rank_tokens [R];
 * with topk_next, local[2] = next-layer slots on the predicted rank / on the
 * source rank.  key_rank [E] nullable (contiguous). */
int oracle_predict(const oracle_cfg* c, const int32_t* topk_cur, const int32_t* trans, const int32_t* count_cur,
                   const int32_t* key_rank, const int32_t* topk_next, int32_t* pred, int32_t* rank_tokens,
                   int64_t* local);

/* Replica slots [TopoEP 3.2]: slot_expert / slot_main [R][N_slot] (-1 empty),
 * inst_slot [E+B]; the parameter pull replica_params[r][j] = main_params[e]
 * ([R][N_slot][P] from [E][P]) and the gradient return
 * grad_accum[main(e)][r][e - main(e)*E/R] = replica_grads[r][j] ([R][R][E/R][P]). */
int oracle_slot_map(const oracle_cfg* c, int32_t n_inst, const int32_t* inst_expert, const int32_t* inst_rank,
                    int32_t* slot_expert, int32_t* slot_main, int32_t* inst_slot);
int oracle_replica_pull(const oracle_cfg* c, const int32_t* slot_expert, const uint16_t* main_params, int64_t P,
                        uint16_t* replica_params);
int oracle_replica_push(const oracle_cfg* c, const int32_t* slot_expert, const uint16_t* replica_grads, int64_t P,
                        uint16_t* grad_accum);

#ifdef __cplusplus
}
#endif
#endif
