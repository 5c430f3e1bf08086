"""The oracle's pins catch plausible mistakes in the oracle itself.

Each case below plants one slip in a temporary copy of the oracle's C
source (a wrong head -> group map, a block-table lookup skipped, a dropped
term, a wrong scale or rounding, an off-by-one in the budget or the partial
page), builds it with gcc, and runs the pins of ``test_oracle_pins.py``
against that build in a child process.  The pins must fail for every
mutant.  The regression fixture of the tiny workload is not run here: it
holds values the oracle wrote itself, so it does not count as a pin.

Everything happens on the CPU; the product library is not involved.
"""
import concurrent.futures
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "locks_oracle.c")

# (name, text in the oracle, replacement)
MUTANTS = [
    ("scan: head h = hh*H + g instead of g*G + hh",
     "        const int h = g * G + hh;\n        widen((size_t)d, q + ((size_t)b * L->num_q_heads + h)"
     " * d, qh);\n        est[hh] = orc_page_estimate",
     "        const int h = hh * H + g;\n        widen((size_t)d, q + ((size_t)b * L->num_q_heads + h)"
     " * d, qh);\n        est[hh] = orc_page_estimate"),
    ("scan: unit read from logical page, block table skipped",
     "    const size_t unit = (size_t)L->block_table[(size_t)b * L->max_pages + j] * H + g;\n"
     "    double* m = ",
     "    const size_t unit = (size_t)j * H + g;\n    double* m = "),
    ("scan: per-head output written to another head's row",
     "head_mass[((size_t)b * L->num_q_heads + g * G + hh) * MP + j] = est[hh];",
     "head_mass[((size_t)b * L->num_q_heads + hh * H + g) * MP + j] = est[hh];"),
    ("share: head h = hh*H + g instead of g*G + hh",
     "                        const int h = g * G + hh;\n                        terms[hh]",
     "                        const int h = hh * H + g;\n                        terms[hh]"),
    ("share: head total over one page too few",
     "z[h] = orc_lse(full, head_mass",
     "z[h] = orc_lse(full > 1 ? full - 1 : full, head_mass"),
    ("share: log G dropped from the mean",
     "v = orc_lse(G, terms) - log((double)G);", "v = orc_lse(G, terms);"),
    ("exact: head h = hh*H + g instead of g*G + hh",
     "            const int h = g * G + hh;\n            widen((size_t)d, q + ((size_t)b * "
     "L->num_q_heads + h) * d, qh);\n            est[hh] = orc_page_exact_lse",
     "            const int h = hh * H + g;\n            widen((size_t)d, q + ((size_t)b * "
     "L->num_q_heads + h) * d, qh);\n            est[hh] = orc_page_exact_lse"),
    ("build: centroid divided by P - 1",
     "        mu[e] = s / P;\n    }\n    /* centred", "        mu[e] = s / (P - 1);\n    }\n    /* centred"),
    ("build: singular values sorted ascending",
     "while (k > 0 && norms[order[k - 1]] < norms[oi])",
     "while (k > 0 && norms[order[k - 1]] > norms[oi])"),
    ("build: coefficients of the uncentred keys",
     "dot(d, vk, kc + (size_t)i * d);", "dot(d, vk, keys + (size_t)i * d);"),
    ("build: null directions kept",
     "const int null_dir = !(s > tiny);", "const int null_dir = 0 * (s > tiny);"),
    ("build pool: written to the logical page's block",
     "const size_t unit = (size_t)L->block_table[(size_t)b * L->max_pages + j] * H + g;\n"
     "            for (int e = 0; e < d; ++e) mu[unit",
     "const size_t unit = (size_t)j * H + g;\n            for (int e = 0; e < d; ++e) mu[unit"),
    ("estimate: logits scaled by 1/d",
     "    const double scale = 1.0 / sqrt((double)d);\n    for (int i = 0; i < P; ++i) logit[i]",
     "    const double scale = 1.0 / (double)d;\n    for (int i = 0; i < P; ++i) logit[i]"),
    ("estimate: centroid term dropped",
     "const double qmu = dot(d, q, mu);", "const double qmu = 0.0 * dot(d, q, mu);"),
    ("estimate: coefficients read transposed",
     "logit[i] = (qmu + dot(r, t, coef + (size_t)i * r)) * scale;",
     "{ double s_ = 0; for (int k = 0; k < r; ++k) s_ += t[k] * coef[(size_t)k * P + i]; "
     "logit[i] = (qmu + s_) * scale; }"),
    ("estimate: basis read transposed",
     "for (int k = 0; k < r; ++k) t[k] = dot(d, basis + (size_t)k * d, q); /* V_j^T q */",
     "for (int k = 0; k < r; ++k) { t[k] = 0; for (int e = 0; e < d; ++e) "
     "t[k] += basis[(size_t)e * r + k] * q[e]; }"),
    ("lse: no max shift",
     "    for (int i = 0; i < n; ++i) s += exp(x[i] - m);\n    return m + log(s);",
     "    for (int i = 0; i < n; ++i) s += exp(x[i]);\n    return log(s);"),
    ("select: ties to the higher page",
     "return (x->page > y->page) - (x->page < y->page);\n}\n\nstatic int cmp_page",
     "return (x->page < y->page) - (x->page > y->page);\n}\n\nstatic int cmp_page"),
    ("select: winners not put in page order",
     "    qsort(all, (size_t)k, sizeof(ranked_t), cmp_page);\n", ""),
    ("select: budget rounded up to whole pages",
     "const int k = budget_tokens / L->page_size;",
     "const int k = (budget_tokens + L->page_size - 1) / L->page_size;"),
    ("attend: partial last page left out",
     "            for (int j = cand; j < np; ++j) pages[n_pages++] = j;",
     "            for (int j = cand; j < full_pages(L, b); ++j) pages[n_pages++] = j;"),
    ("attend: head -> group by h % H",
     "const int b = (int)(bh / Hq), h = (int)(bh % Hq), g = h / G;",
     "const int b = (int)(bh / Hq), h = (int)(bh % Hq), g = h % H;"),
    ("attend: list entries that are not candidates accepted",
     "if (s[t] >= 0 && s[t] < cand) pages[n_pages++] = s[t];",
     "if (s[t] >= 0 && s[t] <= cand) pages[n_pages++] = s[t];"),
    ("select: pages without a summary compete",
     "            orc_select_topk(candidate_pages(L, b), page_mass + row * MP, k, width,",
     "            orc_select_topk(full_pages(L, b), page_mass + row * MP, k, width,"),
    ("scan: pages without a summary scanned",
     "        if (j < candidate_pages(L, b)) {\n            a = scan_unit(",
     "        if (j < full_pages(L, b)) {\n            a = scan_unit("),
    ("attend: full pages without a summary left out",
     "            for (int j = cand; j < np; ++j) pages[n_pages++] = j;",
     "            for (int j = full_pages(L, b); j < np; ++j) pages[n_pages++] = j;"),
    ("quantise: ties rounded away from zero",
     "const float y = rintf(x[(size_t)i * stride] / s);",
     "const float y = roundf(x[(size_t)i * stride] / s);"),
    ("dequantise: int4 nibble read without sign",
     "return v >= 8 ? v - 16 : v;", "return v;"),
    ("dequantise: coefficient column uses the basis row's scale",
     "(float)((double)sc[1 + r + k] * coef_q[(u * P + t) * r + k]);",
     "(float)((double)sc[1 + k] * coef_q[(u * P + t) * r + k]);"),
    ("sketch: unit written to the logical page's block",
     "const size_t unit = (size_t)L->block_table[(size_t)b * L->max_pages + j] * H + g;\n"
     "                double mu[1024];",
     "const size_t unit = (size_t)j * H + g;\n                double mu[1024];"),
    ("covariance: keys not centred",
     "for (int e = 0; e < d; ++e) kc[(size_t)i * d + e] = k[(size_t)i * d + e] - mu[e];",
     "for (int e = 0; e < d; ++e) kc[(size_t)i * d + e] = k[(size_t)i * d + e];"),
]


def _run_pins_against(name, old, new, tmpdir):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site not unique or missing: {name}"
    tag = "m%08x" % (abs(hash(name)) & 0xFFFFFFFF)
    csrc = os.path.join(tmpdir, tag + ".c")
    so = os.path.join(tmpdir, tag + ".so")
    with open(csrc, "w") as f:
        f.write(src.replace(old, new))
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-I",
                           os.path.join(ROOT, "oracle"), "-o", so, csrc, "-lm"])
    code = ("import sys; sys.path.insert(0, %r); import oracle; oracle._LIB_PATH = %r; "
            "import pytest; sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', "
            "'-o', 'addopts=', %r]))" % (ROOT, so, os.path.join(HERE, "test_oracle_pins.py")))
    env = dict(os.environ, OMP_NUM_THREADS="2")
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT,
                         env=env, timeout=600)
    failed = [ln for ln in res.stdout.splitlines() if ln.startswith("FAILED")]
    return name, res.returncode, failed


def test_every_planted_mistake_fails_a_pin(tmp_path):
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(lambda m: _run_pins_against(*m, str(tmp_path)), MUTANTS))
    survivors = [name for name, rc, _ in results if rc == 0]
    for name, rc, failed in results:
        print(f"{name}: exit {rc}, first failure {failed[:1]}")
    assert not survivors, f"mutants not caught by any pin: {survivors}"


def test_unmutated_oracle_passes_the_pins(tmp_path):
    name, rc, failed = _run_pins_against("none", "#include <math.h>", "#include <math.h>",
                                         str(tmp_path))
    assert rc == 0, failed
