"""Plant mistakes in copies of oracle.c (on the CPU) and check that the pins
catch each one: a dropped term, a wrong sign or index, an off-by-one edge, a
transposed operand.  A mutant that passes every pin would mean the pins leave
that part of the oracle unchecked."""
import json
import os
import subprocess
import sys
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "mean_divisor": ("out[e] /= (double)(t1 - t0);", "out[e] /= (double)(t1 - t0 + 1);"),
    "l2_no_normalise": ("scale = ss > 0.0 ? 1.0 / sqrt(ss) : 0.0;", "scale = 1.0;"),
    "compress_head0": ("int64_t row = ((cu_k[b] + t) * h_kv + c) * (int64_t)d;",
                       "int64_t row = ((cu_k[b] + t) * h_kv) * (int64_t)d;"),
    "score_drops_head": ("for (int hh = 0; hh < G; hh++)\n            for (int e = 0; e < d; e++)\n"
                         "                qs[e] += qh[hh * d + e];",
                         "for (int hh = 0; hh < G - 1; hh++)\n            for (int e = 0; e < d; e++)\n"
                         "                qs[e] += qh[hh * d + e];"),
    "score_wrong_block": ("kv[e] = k_cmp[(((int64_t)c * batch + b) * nb_max + j) * d + e];",
                          "kv[e] = k_cmp[(((int64_t)c * batch + b) * nb_max + (j > 0 ? j - 1 : j)) * d + e];"),
    "overlap_ignored": ("int64_t t0 = j * g - overlap,", "int64_t t0 = j * g,"),
    "overlap_forward": ("t1 = (j + 1) * (int64_t)g;\n        double *out", "t1 = (j + 1) * (int64_t)g + overlap;\n        double *out"),
    "max_is_sum": ("cs[nc].s = mode == OR_SEL_MAX ? best / sqrt((double)d) : dot / sqrt((double)d);",
                   "cs[nc].s = dot / sqrt((double)d);"),
    "max_takes_min": ("else if (dh > best)", "else if (dh < best || best == -INFINITY)"),
    "softmax_no_tau": ("lg[nc * G + hh] = dh / tau;", "lg[nc * G + hh] = dh;"),
    "softmax_unshifted_sum": ("z += exp(lg[x * G + hh] - m);", "z += exp(lg[x * G + hh]);"),
    "attn_no_lse": ("cs[x].s += exp(lgt[t] - lse_ih);", "cs[x].s += exp(lgt[t] - m);"),
    "attn_causal_short": ("for (int64_t t = 0; t <= p_i; t++)\n                        z += exp(lgt[t] - m);",
                          "for (int64_t t = 0; t < p_i; t++)\n                        z += exp(lgt[t] - m);"),
    "attn_block_first_token": ("int64_t t0 = (int64_t)cs[x].j * g, t1 = t0 + g - 1;",
                               "int64_t t0 = (int64_t)cs[x].j * g, t1 = t0;"),
    "attn_last_query_only": ("for (int64_t i = qa; i < qb; i++) {\n                int64_t p_i",
                             "for (int64_t i = qb - 1; i < qb; i++) {\n                int64_t p_i"),
    "ward_unweighted": ("return (double)na * nb / (na + nb) * dist2;", "return dist2;"),
    "ward_sums_not_means": ("const double diff = sa[e] / na - sb[e] / nb;", "const double diff = sa[e] - sb[e];"),
    "ward_not_mutual": ("if (alive[a] && nn[a] > a && nn[nn[a]] == a)", "if (alive[a] && nn[a] > a)"),
    "ward_truncate_dearest": ("(nnc[pa[y]] < nnc[pa[y - 1]] ||", "(nnc[pa[y]] > nnc[pa[y - 1]] ||"),
    "ward_ignore_cap": ("if (o == a || !alive[o] || size[a] + size[o] > capg)", "if (o == a || !alive[o])"),
    "centroid_unnormalised": ("cen[(int64_t)nbk * d + e] = nrm > 0.0 ? S[a * d + e] / nrm : 0.0;",
                              "cen[(int64_t)nbk * d + e] = S[a * d + e];"),
    "bucket_blocks_off_by_one": ("int64_t ncb = (p_sel + 1) / C;", "int64_t ncb = (p_sel + 1 + C - 1) / C;"),
    "expand_keeps_window": ("if (!(grp * g < p_sel - window + 1 && (grp + 1) * g > n_init))",
                            "if (!((grp + 1) * g > n_init))"),
    "expand_drops_member": ("for (int x = off[lb]; x < off[lb + 1]; x++) {", "for (int x = off[lb]; x < off[lb + 1] - 1; x++) {"),
    "softmax_one_head": ("for (int hh = 0; hh < G; hh++) {\n                double m = -INFINITY, z = 0.0;",
                         "for (int hh = 0; hh < 1; hh++) {\n                double m = -INFINITY, z = 0.0;"),
    "ties_to_higher": ("return (x->j > y->j) - (x->j < y->j);", "return (x->j < y->j) - (x->j > y->j);"),
    "ascending_scores": ("if (x->s > y->s)\n        return -1;", "if (x->s < y->s)\n        return -1;"),
    "visibility_off_by_one": ("if (t1 > p_sel)\n                continue;", "if (t1 > p_sel + 1)\n                continue;"),
    "fixed_window_off_by_one": ("return t < n_init || t >= p_sel - window + 1;",
                                "return t < n_init || t >= p_sel - window;"),
    "attend_window_off_by_one": ("int member = t < n_init || t >= p_sel - window + 1 || sel[t / g];",
                                 "int member = t < n_init || t >= p_sel - window + 2 || sel[t / g];"),
    "attend_init_short": ("int member = t < n_init || t",
                          "int member = t < n_init - 1 || t"),
    "shared_psel": ("p_sel = first_query_pos(b, cu_q, cu_k, q_pos0) - 1;",
                    "p_sel = first_query_pos(b, cu_q, cu_k, q_pos0);"),
    "no_scale": ("logit[t] = scale * dot;", "logit[t] = dot;"),
    "logit_uses_v": ("dot += elem(q, dtype, qoff + e) * elem(k, dtype, koff + e);",
                     "dot += elem(q, dtype, qoff + e) * elem(v, dtype, koff + e);"),
    "wrong_kv_head": ("int h = req_h[r], c = h / G;", "int h = req_h[r], c = h % h_kv;"),
    "unweighted_v": ("o[e] += wgt * elem(v, dtype, voff + e);", "o[e] += elem(v, dtype, voff + e);"),
}

RUNNER = r"""
import json, sys
sys.path[:0] = [sys.argv[1], sys.argv[2]]
import pins
failed = []
for p in pins.ALL:
    try:
        p()
    except Exception as e:
        failed.append(p.__name__)
print(json.dumps(failed))
"""


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    find, repl = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(find) == 1, f"mutation site not unique/present: {name}"
    mut = tmp_path / "oracle_mut.c"
    mut.write_text(src.replace(find, repl))
    so = tmp_path / "liboracle_mut.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", str(so),
                           str(mut), "-lm"])
    env = dict(os.environ, ORACLE_LIB=str(so), OMP_NUM_THREADS="4")
    out = subprocess.run([sys.executable, "-c", RUNNER, ROOT, HERE], env=env, capture_output=True,
                         text=True, timeout=300)
    assert out.returncode == 0, out.stderr[-2000:]
    failed = json.loads(out.stdout.strip().splitlines()[-1])
    assert failed, f"mutant {name} passed every pin"
