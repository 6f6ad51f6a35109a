"""The oracle pins are sensitive: each plausible mistake planted in a copy of
the oracle's C source (a dropped term, a wrong index, a flipped comparison)
makes the pin suite fail.  Everything here runs on the CPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "tv_oracle.c")

MUTANTS = {
    "gqa_map_modulo": ("int g = h / (a->hq / a->hkv);", "int g = h % a->hkv;"),
    "scale_dropped": ("scores[p] = a->scale * orc_dot(", "scores[p] = orc_dot("),
    "no_self_attention": ("for (int j = i; j != -1; j = par[j]) vis[j] = 1;",
                          "for (int j = par[i]; j != -1; j = par[j]) vis[j] = 1;"),
    "prefix_off_by_one": ("int visible = p < P || vis[p - P];",
                          "int visible = p < P - 1 || (p >= P && vis[p - P]);"),
    "lse_missing_max": ("  *lse = m + log(l);\n}\n\n/* Path-gather", "  *lse = log(l);\n}\n\n/* Path-gather"),
    "page_slot_swapped": ("int slot = pos % a->page;", "int slot = pos / a->page;"),
    "match_own_target": ("if (dr[j] != tg[par[j]]) ok = 0;", "if (dr[j] != tg[j]) ok = 0;"),
    "tie_to_largest_index": ("if (ok && dep > best_depth)", "if (ok && dep >= best_depth)"),
    "depth_off_by_one": ("      int d = -1;\n", "      int d = 0;\n"),
    "anchor_depth_reset": ("branch_depth[n0 + i] = branch_depth[n0 + i - 1] + 1;",
                           "branch_depth[n0 + i] = 1;"),
    "dcut_tie_to_larger_request": ("if (a->b != c->b) return a->b < c->b ? -1 : 1;",
                                   "if (a->b != c->b) return a->b > c->b ? -1 : 1;"),
    "dcut_roots_not_reserved": ("for (int r = 0; r < budget - batch; ++r)",
                                "for (int r = 0; r < budget - batch - 1; ++r)"),
    "dcut_no_upper_clamp": ("      if (c > 1.0f) c = 1.0f;\n", ""),
    "dcut_score_ascending": ("if (a->s != c->s) return a->s > c->s ? -1 : 1;",
                             "if (a->s != c->s) return a->s < c->s ? -1 : 1;"),
    "second_root_accepted": ("if (par[i] < 0 || par[i] >= i) return 1;",
                             "if (par[i] < -1 || par[i] >= i) return 1;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_oracle_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation anchor not found: " + name
    mut = tmp_path / "mutant.c"
    mut.write_text(src.replace(old, new))
    lib = tmp_path / "mutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", str(mut), "-o", str(lib), "-lm"])
    env = dict(os.environ, TV_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, "pins did not catch mutant %s:\n%s" % (name, r.stdout[-2000:])


# Mistakes planted in a copy of the oracle's Python front end (the E2E-TV
# statistics are written there, in numpy); the copy is imported as `oracle`
# before the pins run.
PY_SRC = os.path.join(ROOT, "oracle", "oracle.py")
PY_MUTANTS = {
    "sampled_residual_not_clamped": ("r = np.maximum(p - q, 0.0)", "r = p - q"),
    "sampled_rejected_token_kept_in_q": ("                q[x] = 0.0\n", ""),
    "sampled_accept_when_above": ("                if lhs < rhs:", "                if lhs > rhs:"),
    "sampled_bonus_from_unreduced_target": ("                cdf = np.cumsum(p)",
                                            "                cdf = np.cumsum(_dist(tl[lo + node], T))"),
    "sampled_residual_after_q_update": ("                r = np.maximum(p - q, 0.0)\n                if r.sum() > 0:\n                    p = r / r.sum()\n                q = q.copy()\n                q[x] = 0.0\n                if q.sum() > 0:\n                    q = q / q.sum()\n",
                                        "                q = q.copy()\n                q[x] = 0.0\n                if q.sum() > 0:\n                    q = q / q.sum()\n                r = np.maximum(p - q, 0.0)\n                if r.sum() > 0:\n                    p = r / r.sum()\n"),
    "e2e_max_instead_of_min": ("alpha[i] = np.minimum(p, q).sum()", "alpha[i] = np.maximum(p, q).sum() - 1.0"),
    "e2e_no_temperature": ("d = _np(draft_logits, np.float64) / float(temperature)",
                           "d = _np(draft_logits, np.float64)"),
    "e2e_prefix_not_reset": ("        run = 1.0\n", ""),
    "graft_parent_is_previous_node": ("src = int(root) if par[j] < 0 else int(out[b, par[j]])",
                                      "src = int(root) if par[j] < 0 else int(out[b, j - 1])"),
    "graft_rank_ignored": ("t = int(adj[src, rank[j]])", "t = int(adj[src, 0])"),
    "graft_first_writer_wins": ("    for i in range(len(tok)):              # in node order: a later node overwrites",
                                "    for i in reversed(range(len(tok))):"),
    "graft_ties_to_larger_id": ("order = np.lexsort((ids, -key))", "order = np.lexsort((-ids, -key))"),
    "e2e_expected_counts_root": ("            expected[b] += run", "            expected[b] += run + (i == int(cu[b]))"),
}


def _run_pins_with_python_oracle(tmp_path, old=None, new=None):
    """Run the E2E-TV, Graft and sampled-acceptance pins against a copy of the oracle package (optionally
    mutated); returns pytest's exit code (0 all passed, 1 some failed)."""
    import shutil
    pkg = tmp_path / "oracle"
    shutil.copytree(os.path.join(ROOT, "oracle"), pkg,
                    ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    if old is not None:
        src = (pkg / "oracle.py").read_text()
        assert src.count(old) >= 1, "mutation anchor not found"
        (pkg / "oracle.py").write_text(src.replace(old, new))
    code = ("import sys, importlib.util\n"
            "spec = importlib.util.spec_from_file_location('oracle', %r, submodule_search_locations=[%r])\n"
            "m = importlib.util.module_from_spec(spec); sys.modules['oracle'] = m; spec.loader.exec_module(m)\n"
            "import pytest\n"
            "sys.exit(pytest.main(['-x', '-q', '-p', 'no:cacheprovider', '-k', 'e2e or graft or sampled', %r]))\n"
            % (str(pkg / "__init__.py"), str(pkg), os.path.join(ROOT, "tests", "test_oracle_pins.py")))
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    return r.returncode, r.stdout


def test_python_oracle_copy_passes_unmutated(tmp_path):
    rc, out = _run_pins_with_python_oracle(tmp_path)
    assert rc == 0, out[-2000:]


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_planted_python_oracle_mistake_is_caught(name, tmp_path):
    rc, out = _run_pins_with_python_oracle(tmp_path, *PY_MUTANTS[name])
    assert rc == 1, "pins did not catch mutant %s (exit %d):\n%s" % (name, rc, out[-2000:])
