"""The oracle's pins catch plausible mistakes: each case plants one mistake
(a dropped term, a wrong index or operand, an off-by-one) in a temporary copy
of the oracle and runs the oracle's pin tests (tests/test_oracle.py) against
that copy in a child process; at least one pin must fail.  The oracle itself
is not modified."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# name: (text of the oracle, the mistake put in its place)
MUTATIONS = {
    "decode_gqa_interleaved": ("        hs = [h for h in heads if h // group == g]",
                               "        hs = [h for h in heads if h % hkv == g]"),
    "prefill_gqa_interleaved": ("            if h // group != g:", "            if h % hkv != g:"),
    "scale_dropped": ("    s = (q @ k.T) * float(scale)\n    if last_pos", "    s = (q @ k.T)\n    if last_pos"),
    "causal_mask_strict": ("        s = np.where(j <= np.asarray(last_pos)[:, None], s, -np.inf)",
                           "        s = np.where(j < np.asarray(last_pos)[:, None], s, -np.inf)"),
    "prefill_top_left_aligned": ("    last = ctx - qlen + rows", "    last = rows"),
    "prefill_position_off_by_one": ("    last = ctx - qlen + rows", "    last = ctx - qlen + rows - 1"),
    "store_row_and_block_swapped": ("        blk, row = divmod(s, bs)", "        row, blk = divmod(s, bs)"),
    "store_k_written_into_v": ("        v_pool[blk, :, row, :] = v_new[i]", "        v_pool[blk, :, row, :] = k_new[i]"),
    "store_negative_slot_written": ("        if s < 0:\n            continue\n        blk, row", "        blk, row"),
    "gather_ignores_block_table": ("        phys = int(table_row[lb])", "        phys = lb"),
    "gather_k_chunks_transposed": ("        k[lo:hi] = kb.transpose(2, 0, 1, 3).reshape(rows, hkv, d)",
                                   "        k[lo:hi] = kb.transpose(2, 0, 3, 1).reshape(rows, hkv, d)"),
    "merge_sum_unweighted": ("    big_l = sum(w[i] * parts[i][1] for i in range(len(parts)))",
                             "    big_l = sum(parts[i][1] for i in range(len(parts)))"),
    "copy_blocks_skips_v": ("        v_pool[dst] = v_pool[src]", "        pass"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_fails_a_pin(name, tmp_path):
    old, new = MUTATIONS[name]
    for d in ("tests", "workloads", "oracle"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d, ignore=shutil.ignore_patterns("__pycache__"))
    shutil.copy(os.path.join(ROOT, "pytest.ini"), tmp_path)
    src_path = tmp_path / "oracle" / "paged_attention.py"
    src = src_path.read_text()
    assert src.count(old) == 1, f"{name}: the oracle text to replace is not unique or not found"
    src_path.write_text(src.replace(old, new))
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle.py", "-q", "-p", "no:cacheprovider"],
                       cwd=tmp_path, capture_output=True, text=True, timeout=300)
    assert r.returncode == 1 and "failed" in r.stdout.splitlines()[-1], (
        f"{name}: no pin failed\n{r.stdout[-2000:]}\n{r.stderr[-2000:]}")
