/*
 * Seeded synthetic inputs for the MoE dispatch-planning path.
 *
 * This file holds only random-number generation and the workload recipe
 * (gate logits and bf16 hidden states).  It contains none of the planning
 * arithmetic: both the CPU oracle and the HIP path read the buffers it
 * writes, and neither links it.
 *
 * Workload model
 *   - TopoEP (section 6.4, "Sensitivity to routing skew") draws random gate
 *     logits plus a fixed expert-specific bias; a stronger bias concentrates
 *     the load on fewer experts.  The bias here is a Zipf law over a seeded
 *     expert permutation: bias[e] = -s * ln(1 + rank(e)), i.e. the log of the
 *     Zipf weight (rank+1)^-s.
 *   - "Expert Coupling in MoE Pretraining" (sections "Experts Are Correlated
 *     Within a Layer" and "Routing Is Also Correlated Across Layers") reports
 *     co-selected expert groups and layer-to-layer routing structure.  A token
 *     draws a latent group of experts that all get a boost beta; across layers
 *     the group follows a seeded map with probability p, else it is redrawn.
 *
 * Random numbers: SplitMix64 (Steele, Lea, Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) used as a counter-based
 * generator: draw(stream, i) = mix64(base(stream) + (i + 1) * gamma).
 * Uniforms are ((x >> 11) + 0.5) * 2^-53, normals come from the Box-Muller
 * transform in double precision (cos branch for even i, sin branch for odd i).
 */
#include <stdint.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t synth_stream_base(uint64_t seed, uint64_t stream) {
  return mix64(mix64(seed + GAMMA) ^ mix64(stream * 0xD1B54A32D192ED03ULL + GAMMA));
}

static inline uint64_t draw(uint64_t base, uint64_t i) { return mix64(base + (i + 1) * GAMMA); }

static inline double uni(uint64_t x) { return ((double)(x >> 11) + 0.5) * (1.0 / 9007199254740992.0); }

/* Unbiased-enough bounded integer in [0, n): multiply-shift of a 64-bit draw. */
static inline uint32_t below(uint64_t x, uint32_t n) {
  return (uint32_t)(((unsigned __int128)x * n) >> 64);
}

static inline double normal_at(uint64_t base, uint64_t i) {
  uint64_t pair = i >> 1;
  double u1 = uni(draw(base, 2 * pair));
  double u2 = uni(draw(base, 2 * pair + 1));
  double r = sqrt(-2.0 * log(u1));
  double th = 6.283185307179586 * u2;
  return (i & 1) ? r * sin(th) : r * cos(th);
}

/* Stream ids: one per tensor kind and layer. */
enum { ST_NOISE = 0, ST_ZIPF_PERM = 1, ST_GROUP_PERM = 2, ST_GROUP_DRAW = 3,
       ST_GROUP_MAP = 4, ST_COUPLE_COIN = 5, ST_HIDDEN = 6, ST_KINDS = 16 };

static uint64_t sbase(uint64_t seed, int layer, int kind) {
  return synth_stream_base(seed, (uint64_t)layer * ST_KINDS + (uint64_t)kind);
}

/* Seeded Fisher-Yates permutation of 0..n-1 (out[pos] = item). */
void synth_permutation(uint64_t seed, int layer, int kind, int32_t n, int32_t* out) {
  uint64_t b = sbase(seed, layer, kind);
  for (int32_t i = 0; i < n; ++i) out[i] = i;
  for (int32_t i = n - 1; i > 0; --i) {
    uint32_t j = below(draw(b, (uint64_t)i), (uint32_t)i + 1);
    int32_t tmp = out[i]; out[i] = out[j]; out[j] = tmp;
  }
}

/*
 * Latent group of each token for each layer: g[l*T + t] in [0, ngroups).
 * Layer 0 is uniform.  Layer l+1 keeps phi_l(g) with probability couple_p
 * (phi_l a seeded permutation of the groups), else redraws uniformly.
 * couple_p = 0 gives independent layers.
 */
void synth_groups(uint64_t seed, int64_t T, int32_t ngroups, int32_t L, double couple_p, int32_t* g) {
  int32_t* phi = (int32_t*)malloc(sizeof(int32_t) * (size_t)ngroups);
  for (int32_t l = 0; l < L; ++l) {
    uint64_t bd = sbase(seed, l, ST_GROUP_DRAW);
    uint64_t bc = sbase(seed, l, ST_COUPLE_COIN);
    if (l > 0) synth_permutation(seed, l - 1, ST_GROUP_MAP, ngroups, phi);
    for (int64_t t = 0; t < T; ++t) {
      int32_t fresh = (int32_t)below(draw(bd, (uint64_t)t), (uint32_t)ngroups);
      int32_t v = fresh;
      if (l > 0 && uni(draw(bc, (uint64_t)t)) < couple_p) v = phi[g[(int64_t)(l - 1) * T + t]];
      g[(int64_t)l * T + t] = v;
    }
  }
  free(phi);
}

/*
 * Gate logits of one layer, f32 [T, E] row-major:
 *   logit = f32( z + zipf_bias(e) + (e in group(t) ? beta : 0) ),  z ~ N(0,1).
 * zipf_s <= 0 disables the bias; groups == NULL or beta == 0 disables the boost.
 * The experts of group g are perm[g*group_size .. (g+1)*group_size) of a seeded
 * per-layer permutation.
 */
void synth_logits(uint64_t seed, int32_t layer, int64_t T, int32_t E, double zipf_s,
                  double beta, int32_t group_size, const int32_t* groups, int32_t nthreads, float* out) {
  double* bias = (double*)calloc((size_t)E, sizeof(double));
  int32_t* perm = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  int32_t* group_of = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  if (zipf_s > 0) {
    synth_permutation(seed, layer, ST_ZIPF_PERM, E, perm);
    for (int32_t pos = 0; pos < E; ++pos) bias[perm[pos]] = -zipf_s * log(1.0 + (double)pos);
  }
  int use_groups = (groups != NULL && beta != 0.0 && group_size > 0);
  if (use_groups) {
    synth_permutation(seed, layer, ST_GROUP_PERM, E, perm);
    for (int32_t pos = 0; pos < E; ++pos) group_of[perm[pos]] = pos / group_size;
  }
  uint64_t bn = sbase(seed, layer, ST_NOISE);
  (void)nthreads;
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1)
  for (int64_t t = 0; t < T; ++t) {
    int32_t gt = use_groups ? groups[t] : -1;
    for (int32_t e = 0; e < E; ++e) {
      double v = normal_at(bn, (uint64_t)t * (uint64_t)E + (uint64_t)e) + bias[e];
      if (use_groups && group_of[e] == gt) v += beta;
      out[t * E + e] = (float)v;
    }
  }
  free(bias); free(perm); free(group_of);
}

/* f32 -> bf16, round to nearest even (finite inputs). */
static inline uint16_t bf16_rne(float f) {
  uint32_t u; memcpy(&u, &f, 4);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

/* Hidden states bf16 [T, H] row-major, N(0,1) rounded to f32 then to bf16 (RNE). */
void synth_hidden(uint64_t seed, int64_t T, int64_t H, int32_t nthreads, uint16_t* out) {
  uint64_t b = sbase(seed, 0, ST_HIDDEN);
  int64_t n = T * H;
  (void)nthreads;
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1)
  for (int64_t i = 0; i < n; i += 2) {
    uint64_t pair = (uint64_t)i >> 1;
    double u1 = uni(draw(b, 2 * pair));
    double u2 = uni(draw(b, 2 * pair + 1));
    double r = sqrt(-2.0 * log(u1));
    double th = 6.283185307179586 * u2;
    out[i] = bf16_rne((float)(r * cos(th)));
    if (i + 1 < n) out[i + 1] = bf16_rne((float)(r * sin(th)));
  }
}

/* The f32 normals behind synth_hidden (before the bf16 rounding), for tests. */
void synth_hidden_f32(uint64_t seed, int64_t T, int64_t H, float* out) {
  uint64_t b = sbase(seed, 0, ST_HIDDEN);
  for (int64_t i = 0; i < T * H; ++i) out[i] = (float)normal_at(b, (uint64_t)i);
}

/* Raw 64-bit draws, for tests of the generator itself. */
void synth_draws(uint64_t seed, uint64_t stream, int64_t n, uint64_t* out) {
  uint64_t b = synth_stream_base(seed, stream);
  for (int64_t i = 0; i < n; ++i) out[i] = draw(b, (uint64_t)i);
}
