"""Mutation check of the oracle's pins.

Each entry below plants one plausible mistake (a dropped term, a wrong sign,
index, denominator or tie-break) in a copy of the oracle package and runs the
pins named beside it against that copy; at least one of them must fail.  The
table covers every function of the oracle, so a function whose mistakes no pin
catches shows up here as a failing entry.  The unmodified copy must pass the
same pins.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle")
PINS = os.path.join(HERE, "test_oracle_pins.py")

# (oracle function, text in oracle.py, planted replacement, pins that must catch it)
MUTATIONS = [
    ("token_slots", "within = ((t % g.ct) * g.ch + (h % g.ch)) * g.cw + (w % g.cw)",
     "within = ((t % g.ct) * g.ch + (w % g.cw)) * g.cw + (h % g.ch)", "token_slots_closed_form"),
    ("token_slots", "(h // g.ch) * g.nw + (w // g.cw)", "(h // g.ch) * g.nh + (w // g.cw)",
     "token_slots_closed_form"),
    ("reorder", "out = np.zeros(x.shape[:-2]", "out = np.ones(x.shape[:-2]", "reorder_round_trip"),
    ("unreorder", "return xc[..., token_slots(g), :]", "return xc[..., np.sort(token_slots(g)), :]",
     "reorder_round_trip"),
    ("unreorder_rows", "return xc[..., token_slots(g)]", "return xc[..., np.sort(token_slots(g))]",
     "block_sparse_equals_token_masked_dense or all_blocks_kept_equals_dense"),
    ("real_slots", "m[token_slots(g)] = True", "m[:g.n_real] = True", "real_slot_counts or pool_ignores_pad"),
    ("pool", "return total / real.sum(axis=1)[:, None]", "return total / g.block",
     "pool_equals_coordinate_gather_mean"),
    ("block_scores", "np.swapaxes(kbar, -1, -2)) / math.sqrt(d)", "np.swapaxes(kbar, -1, -2)) / d",
     "block_probs_match_library or coarse_output_is_library"),
    ("block_softmax", "return e / e.sum(axis=-1, keepdims=True)", "return e / (1.0 + e.sum(axis=-1, keepdims=True))",
     "block_probs_match_library"),
    ("ceil_k", "c = math.ceil(k_frac * n - 1e-9)", "c = math.ceil(k_frac * n)", "ceil_k_edges"),
    ("ceil_k", "c = math.ceil(k_frac * n - 1e-9)", "c = round(k_frac * n)", "ceil_k_edges or topk_count"),
    ("rank_order", "return np.lexsort((j, -s_row))", "return np.lexsort((-j, -s_row))",
     "brute_force_with_exact_ties or uniform_row_topp"),
    ("rank_order", "return np.lexsort((j, -s_row))", "return np.lexsort((j, s_row))", "select_matches_brute_force"),
    ("top_p_count", "hit = np.nonzero(cum >= p)[0]", "hit = np.nonzero(cum > p)[0]", "topp_sink_row_worked"),
    ("top_p_count", "if p >= 1.0:\n        return n", "if p > 1.0:\n        return n", "p_one_keeps_every_block"),
    ("select_row", "keep = max(kc, pc)", "keep = min(kc, pc)", "select_matches_brute_force"),
    ("select_row", "kept = np.sort(order[:keep])", "kept = order[:keep]", "select_matches_brute_force"),
    ("_near_tie", "if gap <= NEAR_TIE * scale:", "if gap < 0:", "test_near_tie_flags"),
    ("_near_tie", "close = np.nonzero(np.abs(prefix - p) < NEAR_TIE)[0]", "close = np.nonzero(prefix < 0)[0]",
     "test_near_tie_flags"),
    ("build_mask", "kc_i = k_default if row_budget is None else int(row_budget[b, h, i])", "kc_i = k_default",
     "row_budgets_keep"),
    ("select_rows", "return [select_row(s[i], kc, p, probs[i]) for i in range(s.shape[0])]",
     "return [select_row(s[i], kc, p) for i in range(s.shape[0])][::-1]", "select_rows_matches_brute_force"),
    ("attention_block", "key_slots = key_slots[real[key_slots]]", "key_slots = key_slots",
     "zero_queries_average or block_sparse_equals_token_masked"),
    ("attention_block", "lse[qmask] = (m + np.log(l))[:, 0]", "lse[qmask] = np.log(l)[:, 0]",
     "all_blocks_kept_equals_dense or block_sparse_equals_token_masked"),
    ("attention_block", "o[qmask] = (e @ v) / l", "o[qmask] = (e @ v) / (l + 1e-3)",
     "all_blocks_kept_equals_dense or attention_normalisation"),
    ("sparse_attention", "attention_block(qc[b, h], kc_[b, h], vc[b, h], kept, g, i, scale)",
     "attention_block(qc[b, h], kc_[b, h], vc[b, h], kept, g, min(i + 1, g.nblk - 1), scale)",
     "all_blocks_kept_equals_dense or block_sparse_equals_token_masked"),
    ("dense_attention", "return np.matmul(e, v) / l, (m + np.log(l))[..., 0]",
     "return np.matmul(e, v) / l, np.log(l)[..., 0]", "dense_attention_matches_library"),
    ("dense_attention", "return np.matmul(e, v) / l, (m + np.log(l))[..., 0]",
     "return np.matmul(e, v) / (l + 1.0), (m + np.log(l))[..., 0]", "dense_attention_matches_library"),
    ("coarse_output", "qbar, kbar, vbar = pool(qc, g), pool(kc_, g), pool(vc, g)",
     "qbar, kbar, vbar = pool(qc, g), pool(kc_, g), pool(kc_, g)", "coarse_output"),
    ("expand_blocks", "out[..., ~real_slots(g), :] = 0.0", "out[..., ~real_slots(g), :] *= 1.0",
     "coarse_output_ignores_pads"),
    ("subcube_of_slot", "return ((tt // rt) * (g.ch // rh) + hh // rh) * (g.cw // rw) + ww // rw",
     "return ((tt // rt) * (g.ch // rh) + ww // rw) * (g.cw // rw) + hh // rh",
     "subcube_means_follow or router_matches_coordinate"),
    ("pool_r", "means = np.where(present[..., None], sums / np.maximum(cnt, 1)[..., None], 0.0)",
     "means = np.where(present[..., None], sums / (g.block // G), 0.0)",
     "subcube_means_follow or router_matches_coordinate"),
    ("router_scores", "s = np.where(present[None, :], s, -np.inf)", "s = s + 0.0", "router_matches_coordinate"),
    ("router_scores", "/ pres.sum(axis=1)[:, None]", "/ G", "router_matches_coordinate"),
    ("router_scores", "per_query = p.sum(axis=-1)", "per_query = p.max(axis=-1)",
     "router_with_cube_sized or router_matches_coordinate"),
    ("sparse_attention_backward", "dk[b, h, ys] += scale * (ds.T @ q_h[xs])", "dk[b, h, ys] += ds.T @ q_h[xs]",
     "backward_matches_finite_differences or backward_all_kept"),
    ("sparse_attention_backward", "D = (dO * o).sum(axis=1, keepdims=True)", "D = 0.0",
     "backward_matches_finite_differences or backward_all_kept"),
    ("sparse_attention_backward", "dv[b, h, ys] += p.T @ dO", "dv[b, h, ys] += p.T @ dO * 0.5",
     "backward_invariants or backward_all_kept"),
    ("sparse_attention_backward", "dq[b, h, xs] += scale * (ds @ k_h[ys])", "dq[b, h, xs] += scale * (p @ k_h[ys])",
     "backward_invariants or backward_matches_finite_differences"),
    ("pooled_mass", "out[idx] = p[idx][lut[idx][:counts[idx]]].sum()",
     "out[idx] = p[idx][lut[idx][:max(counts[idx] - 1, 0)]].sum()", "pooled_mass_closed_forms"),
    ("mask_error", "den = np.abs(o[rows]).sum()", "den = np.abs(o_s[b, h, rows]).sum()",
     "error_decomposition_worked_example"),
    ("mask_error", "t[rows] = p[ridx][:, kept[key_blk]].sum(axis=1)",
     "t[rows] = p[ridx][:, ~kept[key_blk]].sum(axis=1)", "mask_error_tau or error_decomposition_worked"),
    ("error_terms", "e_ren = (1.0 - 1.0 / tau) * ((p * m) @ v)", "e_ren = (1.0 - tau) * ((p * m) @ v)",
     "error_decomposition_worked_example or error_terms_with_constant"),
    ("error_terms", "e_drop = (p * (1.0 - m)) @ v", "e_drop = (p * m) @ v",
     "error_decomposition_worked_example or error_terms_with_constant"),
    ("error_terms", "den += np.abs(p @ v).sum()", "den += np.abs((p * m) @ v).sum()",
     "error_decomposition_worked_example or error_terms_with_constant"),
    ("mask_report", "sink = p[..., 0].mean(axis=-1)", "sink = p[..., 0, :].mean(axis=-1)", "mask_report_closed"),
    ("mask_report", "plogp = np.where(p > 0, p * np.log(p), 0.0)", "plogp = np.where(p > 0, p * np.log2(p), 0.0)",
     "mask_report_closed"),
    ("mask_report", "sum(axis=-1) / float(n * n)", "sum(axis=-1) / float(n)", "mask_report_closed"),
    ("group_count", "return -(-nblk // qg)", "return nblk // qg", "pool_groups or build_mask_groups"),
    ("pool_groups", "out[..., a, :] = xc[..., keep, :].sum(axis=-2) / keep.size",
     "out[..., a, :] = xc[..., keep, :].sum(axis=-2) / (hi - lo)", "pool_groups"),
    ("build_mask_groups", "kc = ceil_k(k_frac, n)\n", "kc = ceil_k(k_frac, nq)\n", "build_mask_groups"),
    ("expand_group_lists", "rows = np.arange(nblk) // qg", "rows = np.arange(nblk) % qg", "build_mask_groups"),
    ("sequence_budget", "return rows * ceil_k(k_frac, nblk)", "return ceil_k(k_frac, rows * nblk)",
     "per_sequence_closed_forms"),
    ("per_sequence_counts", "order = np.lexsort((np.arange(flat.size), -flat))",
     "order = np.lexsort((-np.arange(flat.size), -flat))", "per_sequence_counts_match_greedy or near_tie_flags"),
    ("per_sequence_near_tie", "return close.any(axis=1)", "return np.ones(prob.shape[0], dtype=bool)",
     "per_sequence_near_tie_flags"),
    ("per_sequence_near_tie", "if last - first_out > NEAR_TIE * last:", "if last - first_out > 0:",
     "per_sequence_near_tie_flags"),
    ("per_sequence_near_tie", "close = np.abs(prob - last) <= NEAR_TIE * last", "close = np.abs(prob - last) <= 0.1",
     "per_sequence_near_tie_flags"),
    ("build_mask_per_sequence", "total = sequence_budget(n, n, k_frac)", "total = sequence_budget(n, n, k_frac) - 1",
     "build_mask_per_sequence"),
    ("ideal_block_mass", "out[b, h, i] = per_key_block[blk_of == i].mean(axis=0)",
     "out[b, h, i] = per_key_block[blk_of == i].sum(axis=0)", "ideal_block_mass"),
    ("mask_recall", "out[idx] = np.intersect1d(top, lut[idx][:c]).size / c",
     "out[idx] = np.intersect1d(top, lut[idx][:c]).size / counts.shape[-1]", "mask_recall"),
]


def _copy_oracle(dst, old=None, new=None):
    pkg = os.path.join(dst, "oracle")
    os.makedirs(pkg)
    shutil.copy(os.path.join(SRC, "__init__.py"), pkg)
    with open(os.path.join(SRC, "oracle.py")) as f:
        text = f.read()
    if old is not None:
        assert text.count(old) == 1, f"mutation target not unique or missing: {old!r}"
        text = text.replace(old, new)
    with open(os.path.join(pkg, "oracle.py"), "w") as f:
        f.write(text)


def _run_pins(copy_dir, select):
    env = dict(os.environ, SA_ORACLE_COPY_DIR=copy_dir, PYTHONDONTWRITEBYTECODE="1")
    cmd = [sys.executable, "-m", "pytest", PINS, "-q", "-x", "-p", "no:cacheprovider", "-k", select]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-2000:]


def _one(idx):
    func, old, new, select = MUTATIONS[idx]
    with tempfile.TemporaryDirectory(prefix="oracle_mut_") as d:
        _copy_oracle(d, old, new)
        return _run_pins(d, select)


def test_every_oracle_function_has_a_mutation_entry():
    import oracle as O
    import inspect
    funcs = {n for n, f in inspect.getmembers(O, inspect.isfunction) if f.__module__ == "oracle.oracle"}
    covered = {m[0] for m in MUTATIONS}
    assert funcs - covered == set(), f"oracle functions without a planted mistake: {sorted(funcs - covered)}"


def test_unmodified_oracle_passes_the_selected_pins():
    select = " or ".join(f"({m[3]})" for m in MUTATIONS)
    with tempfile.TemporaryDirectory(prefix="oracle_ref_") as d:
        _copy_oracle(d)
        rc, out = _run_pins(d, select)
    assert rc == 0, out


def test_every_planted_mistake_fails_a_pin():
    workers = max(1, min(8, os.cpu_count() or 1))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        results = list(ex.map(_one, range(len(MUTATIONS))))
    survived = []
    for (func, old, new, select), (rc, out) in zip(MUTATIONS, results):
        # 1: some selected pin failed (caught); 0: all passed (survived);
        # anything else (no test selected, collection error) is a broken entry
        if rc != 1:
            survived.append((func, new, select, rc, out[-400:]))
    assert not survived, "\n".join(f"{f}: {n!r} [{s}] rc={rc}\n{o}" for f, n, s, rc, o in survived)
