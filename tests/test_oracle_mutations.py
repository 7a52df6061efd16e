"""The oracle's pins catch plausible mistakes.

Each case plants one mistake (an off-by-one mask, the other alignment, an
interleaved head mapping, a missing max subtraction, a wrong scale, a
document boundary slip, a misplaced block remainder, an ignored reverse
index, a scatter off by one token, and slips in the zigzag metadata: kv
lengths, the local row order, surplus and prefix handling, the late block)
in a temporary copy of ``oracle/`` and
runs the oracle's pin tests against that copy: every mutation must make them
fail.  Nothing in the repository is modified."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTATIONS = [
    ("oracle/attention.py", "keys[None, :] <= (rows[r0:r1, None] + kv_len - q_len)",
     "keys[None, :] < (rows[r0:r1, None] + kv_len - q_len)", "causal mask off by one"),
    ("oracle/attention.py", "keys[None, :] <= (rows[r0:r1, None] + kv_len - q_len)",
     "keys[None, :] <= rows[r0:r1, None]", "top-left causal alignment"),
    ("oracle/attention.py", "k[:, h // g, :]", "k[:, h % k.shape[1], :]", "interleaved GQA mapping for K"),
    ("oracle/attention.py", "v[:, h // g, :]", "v[:, h % v.shape[1], :]", "interleaved GQA mapping for V"),
    ("oracle/attention.py", "p = np.exp(s - m)", "p = np.exp(s)", "no row-max subtraction"),
    ("oracle/attention.py", "/ np.sum(p, axis=1, keepdims=True)",
     "/ (np.sum(p, axis=1, keepdims=True) + 1e-3)", "perturbed normaliser"),
    ("oracle/attention.py", "return 1.0 / math.sqrt(d)", "return 1.0 / d", "wrong default scale"),
    ("oracle/attention.py", "if lo <= q_start + r < hi]", "if lo <= q_start + r <= hi]",
     "packed document boundary off by one"),
    ("oracle/attention.py", "k_global[lo:hi], v_global[lo:hi],", "k_global[0:hi], v_global[0:hi],",
     "packed rows see earlier documents"),
    ("oracle/zigzag_meta.py", "return [base + (1 if j < rem else 0) for j in range(nblocks)]",
     "return [base + (1 if j >= nblocks - rem else 0) for j in range(nblocks)]",
     "block remainder on the last blocks"),
    ("oracle/zigzag_meta.py",
     "kv_len_next = [prefix[b] + 1 + max(t for bb, _j, t in late if bb == b) for b in range(bs)]",
     "kv_len_next = [prefix[b] + min(t for bb, _j, t in late if bb == b) for b in range(bs)]",
     "kv_len_next without its own block"),
    ("oracle/zigzag_meta.py",
     "kv_len_prev = [prefix[b] + 1 + max(t for bb, _j, t in early if bb == b) for b in range(bs)]",
     "kv_len_prev = [1 + max(t for bb, _j, t in early if bb == b) for b in range(bs)]",
     "kv_len_prev without the cached prefix"),
    ("oracle/zigzag_meta.py", "    local = [e + l for e, l in shards]",
     "    local = [[tk for b in range(bs) for tk in of_block[(b, r)] + of_block[(b, nblk - 1 - r)]]\n"
     "             for r in range(cp_size)]",
     "local rows interleaved per sequence"),
    ("oracle/zigzag_meta.py", "    ext[-1] += surplus", "    ext[0] += surplus",
     "surplus tokens to the first sequence"),
    ("oracle/zigzag_meta.py", "prefix = [max(seqs[b] - ext[b], 0) if has_seqs else 0 for b in range(bs)]",
     "prefix = [max(seqs[b], 0) if has_seqs else 0 for b in range(bs)]", "prefix taken as the full length"),
    ("oracle/zigzag_meta.py", "of_block[(b, nblk - 1 - r)]]\n        return early, late",
     "of_block[(b, (nblk - r) % nblk)]]\n        return early, late",
     "late block index shifted"),
    ("oracle/layout.py", "return np.concatenate([chunks[i] for i in meta.cp_reverse_index], axis=0)",
     "return np.concatenate([chunks[i] for i in sorted(meta.cp_reverse_index)], axis=0)",
     "rerange ignores the reverse index"),
    ("oracle/layout.py", "res[page, pos % page_size] = gathered[gathered_row_of_token(meta, b, t)]",
     "res[page, pos % page_size] = gathered[gathered_row_of_token(meta, b, max(0, t - 1))]",
     "scatter off by one token"),
]

PIN_TESTS = ["tests/test_oracle_meta.py", "tests/test_oracle_layout.py", "tests/test_oracle_attention.py"]


def _copy(tmp_path):
    for sub in ("oracle", "tests", "synth"):
        shutil.copytree(os.path.join(ROOT, sub), tmp_path / sub,
                        ignore=shutil.ignore_patterns("__pycache__"))


def _run_pins(cwd):
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *PIN_TESTS],
                          cwd=cwd, capture_output=True, text=True, timeout=600)


def test_unmutated_copy_passes(tmp_path):
    """Control: the same copy without a mutation passes, so a failure below
    is the mutation's doing."""
    _copy(tmp_path)
    run = _run_pins(tmp_path)
    assert run.returncode == 0, run.stdout[-3000:] + run.stderr[-3000:]


@pytest.mark.parametrize("path,old,new,what", MUTATIONS, ids=[m[3] for m in MUTATIONS])
def test_pins_catch_a_planted_mistake(tmp_path, path, old, new, what):
    _copy(tmp_path)
    target = tmp_path / path
    src = target.read_text()
    assert src.count(old) >= 1, f"mutation site not found: {what}"
    target.write_text(src.replace(old, new, 1))
    run = _run_pins(tmp_path)
    assert run.returncode != 0, f"the oracle's pins missed: {what}"
    assert "failed" in run.stdout, run.stdout[-2000:]   # a test failed, not the collection
