"""Self-test of the oracle pins: plant plausible mistakes in copies of the
oracle source, build each on the CPU, and check that the pin suite rejects
every one of them.  The mistakes are the kind a reader might make when
restating the pages: a dropped factor, a flipped tie-break, a swapped index,
a wrong default.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

from oracle import build as obuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.cpp")

# (name, exact text in the oracle, replacement)
MUTANTS = [
    ("topk order reversed", "topk_idx[t * k + j] = order[j];", "topk_idx[t * k + j] = order[k - 1 - j];"),
    ("topk ascending", "return row[a] > row[b]; });", "return row[a] < row[b]; });"),
    ("cooc diagonal kept", "if (a != b) cooc[(int64_t)a * E + b] += 1;", "cooc[(int64_t)a * E + b] += 1;"),
    ("trans transposed", "trans[(int64_t)a * E + b] += 1;", "trans[(int64_t)b * E + a] += 1;"),
    ("omega interleaved sources", "omega[src_of(d, t) * E + e] += 1;", "omega[(t % R) * E + e] += 1;"),
    ("Eq. 9 factor 2 dropped", "int64_t b = 2 * D[m * E + e] * d.S - d.W;", "int64_t b = D[m * E + e] * d.S - d.W;"),
    ("Eq. 9 local experts", "if (dom_of(c, main_of(d, e)) == m) continue;", "if (dom_of(c, main_of(d, e)) != m) continue;"),
    ("stage 1 ascending benefit", "if (a.first != b.first) return a.first > b.first;",
     "if (a.first != b.first) return a.first < b.first;"),
    ("stage 1 ties to higher rank", "if (best < 0 || nrep[r] < nrep[best]) best = r;",
     "if (best < 0 || nrep[r] <= nrep[best]) best = r;"),
    ("even split remainder to the last", "Uer(e, sel[i]) += w / m + (i < w % m ? 1 : 0);",
     "Uer(e, sel[i]) += w / m + (i >= m - w % m ? 1 : 0);"),
    ("routing ignores the source domain", "if (X(e, r) && dom_of(c, r) == dom_of(c, s)) sel.push_back(r);",
     "if (X(e, r) && r == s) sel.push_back(r);"),
    ("Eq. 10 without the half gap", "int64_t delta = std::min(Uer(e, rb), (L[rb] - L[rt]) / 2);",
     "int64_t delta = std::min(Uer(e, rb), (L[rb] - L[rt]));"),
    ("busiest rank ties to higher rank", "if (L[r] > L[rb]) rb = r;", "if (L[r] >= L[rb]) rb = r;"),
    ("refinement prefers the busier target", "else if (L[rt] != blt) better = L[rt] < blt;",
     "else if (L[rt] != blt) better = L[rt] > blt;"),
    ("refinement prefers new replicas", "else if (is_new != bnew) better = is_new < bnew;",
     "else if (is_new != bnew) better = is_new > bnew;"),
    ("refinement ignores the slot limit", "if (is_new && !(nrep[rt] < d.n_slot && rep_dom[m] < Bd)) continue;",
     "if (is_new && !(rep_dom[m] < Bd)) continue;"),
    ("replicas listed before mains", "      if (main_of(d, e) == r) inst_of[e * R + r] = n++;\n    for (int64_t e = 0; e < E; ++e)\n      if (X(e, r) && main_of(d, e) != r) inst_of[e * R + r] = n++;",
     "      if (X(e, r) && main_of(d, e) != r) inst_of[e * R + r] = n++;\n    for (int64_t e = 0; e < E; ++e)\n      if (main_of(d, e) == r) inst_of[e * R + r] = n++;"),
    ("stage 1 most occupied rank", "if (best < 0 || nrep[r] < nrep[best]) best = r;",
     "if (best < 0 || nrep[r] > nrep[best]) best = r;"),
    ("quota sources descending", "      for (int64_t s = 0; s < R; ++s)\n        for (size_t a = 0; a < insts.size(); ++a) {",
     "      for (int64_t s = R - 1; s >= 0; --s)\n        for (size_t a = 0; a < insts.size(); ++a) {"),
    ("quota instances in reverse rank order",
     "      for (int64_t s = 0; s < R; ++s)\n        for (size_t a = 0; a < insts.size(); ++a) {",
     "      for (int64_t s = 0; s < R; ++s)\n        for (size_t a = insts.size(); a-- > 0;) {"),
    ("quota without the same-rank pass", "bool ok = pass == 0 ? (r == s) :", "bool ok = pass == 0 ? (dom_of(c, r) == dom_of(c, s)) :"),
    ("quota without the same-domain pass", ": pass == 1 ? (dom_of(c, r) == dom_of(c, s)) : true;", ": pass == 1 ? true : true;"),
    ("slot walk off by one", "if (run > p) chosen = i;", "if (run >= p) chosen = i;"),
    ("dispatch order not stable", "[&](int32_t a, int32_t b) { return slot_inst[a] < slot_inst[b]; });",
     "[&](int32_t a, int32_t b) { return slot_inst[a] != slot_inst[b] ? slot_inst[a] < slot_inst[b] : a > b; });"),
    ("budget remainder to high domains", "return c->B / d.M + (dom < c->B % d.M ? 1 : 0);",
     "return c->B / d.M + (dom >= d.M - c->B % d.M ? 1 : 0);"),
    ("slots per rank rounded down", "d.n_slot = c->n_slot > 0 ? c->n_slot : (per_dom + c->G - 1) / c->G;",
     "d.n_slot = c->n_slot > 0 ? c->n_slot : per_dom / c->G;"),
    ("expert bytes halved", "d.W = c->W >= 0 ? c->W : 9LL * c->H * c->H / 4;", "d.W = c->W >= 0 ? c->W : 9LL * c->H * c->H / 8;"),
    ("token bytes one byte per element", "d.S = c->S > 0 ? c->S : 2LL * c->H;", "d.S = c->S > 0 ? c->S : 1LL * c->H;"),
    ("combine weights reversed", "acc += w[j] * (double)x;", "acc += w[k - 1 - j] * (double)x;"),
    ("combine without the maximum", "w[j] = std::exp((double)topk_val[t * k + j] - m);",
     "w[j] = std::exp((double)topk_val[t * k + j]);"),
    ("combine not normalised", "for (int64_t j = 0; j < k; ++j) w[j] /= s;", ""),
    ("combine ignores the dispatch positions", "expert_out[(int64_t)slot_pos[t * k + j] * H + h]",
     "expert_out[(t * k + j) * H + h]"),
    ("placement seeds by lowest index", "const int64_t score = m == 0 ? deg[e] : aff[r * E + e];",
     "const int64_t score = m == 0 ? 0 : aff[r * E + e];"),
    ("placement growth ties to higher index", "if (score > best) { best = score; pick = e; }",
     "if (score >= best) { best = score; pick = e; }"),
    ("swap gain without the pair term", "aff[ra * E + b] - aff[rb * E + b] - 2 * C(a, b);",
     "aff[ra * E + b] - aff[rb * E + b];"),
    ("swap update reversed", "aff[ra * E + x] += C(x, bb) - C(x, ba);", "aff[ra * E + x] += C(x, ba) - C(x, bb);"),
    ("swaps of zero gain accepted", "int64_t ba = -1, bb = -1, bg = 0;", "int64_t ba = -1, bb = -1, bg = -1;"),
    ("dedup counts every slot", "if (!seen) {", "if (true) {"),
    ("dedup interleaved ranks", "rank[q] = key / Er;", "rank[q] = key % c->R;"),
    ("dedup layout tokens descending", "    for (int64_t t = 0; t < T; ++t) {\n      uint32_t mask = 0;",
     "    for (int64_t t = T - 1; t >= 0; --t) {\n      uint32_t mask = 0;"),
    ("dedup slot row off by one", "if (mask >> j & 1u) slot_row[t * k + j] = (int32_t)p;",
     "if (mask >> j & 1u) slot_row[t * k + j] = (int32_t)(p + 1 < N ? p + 1 : p);"),
    ("quality counts main instances as replicas", "if (r != main_of(d, e)) out[4] += q;",
     "if (r == main_of(d, e)) out[4] += q;"),
    ("quality same node excludes the source rank", "if (dom_of(c, r) == dom_of(c, s)) out[2] += q;",
     "if (dom_of(c, r) == dom_of(c, s) && r != s) out[2] += q;"),
    ("quality smallest load is a maximum", "out[6] = std::min<int64_t>(out[6], rank_load[r]);",
     "out[6] = std::max<int64_t>(out[6], rank_load[r]);"),
    ("prediction without the count normalisation",
     "P[a * R + r] = count_cur[a] > 0 ? (double)n[r] / (double)count_cur[a] : 0.0;",
     "P[a * R + r] = count_cur[a] > 0 ? (double)n[r] : 0.0;"),
    ("prediction transposed transitions", "for (int64_t b = 0; b < E; ++b) n[rank_of[b]] += trans[a * E + b];",
     "for (int64_t b = 0; b < E; ++b) n[rank_of[b]] += trans[b * E + a];"),
    ("prediction ties to the higher rank", "if (score[r] > score[best]) best = r;", "if (score[r] >= score[best]) best = r;"),
    ("locality counts the predicted rank of the wrong layer", "if (rank_of[b] == best) local[0] += 1;",
     "if (rank_of[topk_cur[t * k + j]] == best) local[0] += 1;"),
    ("slot map counts main instances", "    if (main_of(d, e) == r) continue;\n    if (used[r] >= ns) return -5;",
     "    if (used[r] >= ns) return -5;"),
    ("slot map records the replica's own rank as the source",
     "slot_main[r * ns + used[r]] = (int32_t)main_of(d, e);", "slot_main[r * ns + used[r]] = (int32_t)r;"),
    ("gradient return ignores the source rank",
     "std::memcpy(grad_accum + ((m * R + r) * Er + (e - m * Er)) * P, replica_grads + (r * ns + j) * P,",
     "std::memcpy(grad_accum + ((m * R + 0) * Er + (e - m * Er)) * P, replica_grads + (r * ns + j) * P,"),
]


PIN_SUITES = ["test_oracle_pins.py", "test_oracle_combine.py", "test_oracle_placement.py", "test_oracle_quality.py",
              "test_oracle_predict.py", "test_oracle_slots.py"]


def judge_mutant(workdir, name, old, new):
    """Build the oracle with one planted mistake and run the pin suites against it in a
    process of their own; returns the suites' exit status (0: every pin accepted it)."""
    text = open(SRC).read()
    assert text.count(old) == 1, "mutation site not found: " + name
    os.makedirs(workdir, exist_ok=True)
    src = os.path.join(workdir, "moe_oracle.cpp")
    with open(src, "w") as fh:
        fh.write(text.replace(old, new))
    lib = obuild.build(out=os.path.join(workdir, "libmutant.so"), src=src)
    env = dict(os.environ, MOE_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider"] +
                       [os.path.join(ROOT, "tests", f) for f in PIN_SUITES],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode


@pytest.fixture(scope="module")
def verdicts(tmp_path_factory):
    """Every mutant judged once, several at a time (each build and pin run is a process of
    its own), so the whole self-test takes about a minute instead of several."""
    base = tmp_path_factory.mktemp("mutants")
    workers = max(1, min(8, (os.cpu_count() or 2) - 1))
    with ThreadPoolExecutor(max_workers=workers) as pool:
        futs = {m[0]: pool.submit(judge_mutant, str(base / ("m%02d" % i)), *m) for i, m in enumerate(MUTANTS)}
        return {k: f.result() for k, f in futs.items()}


@pytest.mark.slow
@pytest.mark.parametrize("name", [m[0] for m in MUTANTS])
def test_pins_reject_mutant(verdicts, name):
    assert verdicts[name] != 0, "the pins accept the mutant '%s'" % name
