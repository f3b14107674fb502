"""The oracle's pins catch plausible mistakes: each case plants one mistake
(a dropped term, a wrong index or operand, an off-by-one, a missed count) in
a temporary copy of the oracle and runs the pin tests against that copy in a
child process -- tests/test_oracle.py for the attention oracle, the model
tests of tests/test_block_manager.py for the block-manager model (not its
comparisons with the library, which would only show a difference); at least
one pin must fail.  The oracle itself is not modified."""

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


# the same for the block-manager model
BM_MUTATIONS = {
    "allocate_floor_not_ceiling": ("        need = -(-num_tokens // self.block_size)",
                                   "        need = num_tokens // self.block_size"),
    "allocate_extra_block_at_multiple": ("        need = -(-num_tokens // self.block_size)",
                                         "        need = num_tokens // self.block_size + 1"),
    "copy_on_write_missed_for_two_holders": ("        elif self.ref[blocks[-1]] > 1:",
                                             "        elif self.ref[blocks[-1]] > 2:"),
    "copy_on_write_keeps_old_reference": ("            pair = (blocks[-1], fresh)\n            self._release(blocks[-1])",
                                          "            pair = (blocks[-1], fresh)"),
    "freed_block_never_reused": ("        if self.ref[b] == 0:\n            self.free.append(b)",
                                 "        if self.ref[b] < 0:\n            self.free.append(b)"),
    "free_list_last_in_first_out": ("            self.free.append(b)", "            self.free.appendleft(b)"),
    "fork_does_not_count_holders": ("        for b in blocks:\n            self.ref[b] += 1", "        for b in blocks:\n            pass"),
    "slot_offset_not_wrapped": ("        return blocks[-1] * self.block_size + length % self.block_size, pair",
                                "        return blocks[-1] * self.block_size + length, pair"),
    "batch_failure_keeps_partial_state": ("                self.free, self.ref, self.seqs = saved\n",
                                          "                pass\n"),
}


def _run_pins(tmp_path, oracle_file, old, new, name, test_args):
    for d in ("tests", "workloads", "oracle"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d, ignore=shutil.ignore_patterns("__pycache__"))
    shutil.copy(os.path.join(ROOT, "pytest.ini"), tmp_path)
    src_path = tmp_path / "oracle" / oracle_file
    src = src_path.read_text()
    assert src.count(old) == 1, f"{name}: the oracle text to replace is not unique or not found"
    src_path.write_text(src.replace(old, new))
    # the package (imported by the block-manager tests) from the repository;
    # the working directory, the copy, comes first on the path, so `oracle`
    # is the mutated copy
    env = dict(os.environ, PYTHONPATH=os.pathsep.join([ROOT, os.environ.get("PYTHONPATH", "")]).rstrip(os.pathsep))
    probe = subprocess.run([sys.executable, "-c", "import oracle; print(oracle.__file__)"], cwd=tmp_path, env=env,
                           capture_output=True, text=True, timeout=120)
    assert probe.stdout.strip().startswith(str(tmp_path)), probe.stdout + probe.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", *test_args, "-q", "-p", "no:cacheprovider"],
                       cwd=tmp_path, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 1 and "failed" in r.stdout.splitlines()[-1], (
        f"{name}: no pin failed\n{r.stdout[-2000:]}\n{r.stderr[-2000:]}")


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_fails_a_pin(name, tmp_path):
    old, new = MUTATIONS[name]
    _run_pins(tmp_path, "paged_attention.py", old, new, name, ["tests/test_oracle.py"])


@pytest.mark.parametrize("name", sorted(BM_MUTATIONS))
def test_planted_block_manager_mistake_fails_a_pin(name, tmp_path):
    old, new = BM_MUTATIONS[name]
    _run_pins(tmp_path, "block_manager.py", old, new, name, ["tests/test_block_manager.py", "-k", "model and not library"])
