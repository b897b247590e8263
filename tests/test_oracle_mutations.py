"""Mistakes planted in the oracle, on the CPU.

Each mutation is a plausible slip in the fp64 oracle or the model allocator:
a dropped term, a wrong sign, a wrong or swapped index, an operand in the
wrong place, the wrong end of a queue. The oracle's pins
(test_oracle_pins.py and test_oracle_allocator.py) must fail on every one.
The mutated oracle is a copy in a temporary directory, run in a child
process; the repository's files are not modified. The pins that run are
those of the attention oracle, the model allocator, the FP8 codec and the
prefix-cache model.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_FILES = ("test_oracle_pins.py", "test_oracle_allocator.py",
             "test_oracle_fp8.py", "test_oracle_prefix_cache.py")

MUTATIONS = [
    ("attention.py", "return h // (num_q_heads // num_kv_heads)",
     "return h % num_kv_heads", "grouped-query mapping by modulo"),
    ("attention.py", "    z = scale * (K @ q)\n    w = np.exp(z - z.max())",
     "    z = (K @ q)\n    w = np.exp(z - z.max())", "scale dropped"),
    ("attention.py", "    w = np.exp(z - z.max())\n    return (w @ V) / w.sum()",
     "    w = np.exp(z.max() - z)\n    return (w @ V) / w.sum()",
     "wrong sign in the exponent"),
    ("attention.py", "    return (w @ V) / w.sum()",
     "    return (w @ V) / w.max()", "normaliser dropped"),
    ("attention.py", "return full + (1 if rest else 0)", "return full",
     "floor instead of ceiling"),
    ("attention.py", "logical_block, offset = divmod(int(pos), block_size)",
     "offset, logical_block = divmod(int(pos), block_size)",
     "block and offset swapped"),
    ("attention.py", "return int(table_row[logical_block]) * block_size + offset",
     "return int(table_row[logical_block]) + offset * block_size",
     "slot stride on the wrong index"),
    ("attention.py", "return max(0, min(pos + 1, context_len))",
     "return max(0, min(pos, context_len))", "causal mask off by one"),
    ("attention.py", "        den = den + c * l", "        den = den + l",
     "merge without rescaling the sums"),
    ("attention.py", "        num = num + c * acc", "        num = num + acc",
     "merge without rescaling the outputs"),
    ("attention.py", "        pool[int(dst)] = pool[int(src)]",
     "        pool[int(src)] = pool[int(dst)]", "block copy reversed"),
    ("attention.py", "        pool[blk, off] = rows[r]",
     "        pool[off % pool.shape[0], blk % pool.shape[1]] = rows[r]",
     "scatter with transposed indices"),
    ("attention.py", "        if slot < 0:\n            continue\n", "",
     "padding slot written"),
    ("fp8.py", "    return _VALUES[np.asarray(codes, dtype=np.int64)] * np.asarray(",
     "    return _VALUES[np.asarray(codes, dtype=np.int64)] / np.asarray(",
     "dequantise divides by the scale"),
    ("fp8.py", "    return np.where(nan, nan_codes, out).astype(np.uint8)",
     "    return out.astype(np.uint8)", "NaN stored as a finite code"),
    ("fp8.py", "even = [c for c in tied if (c & 1) == 0]",
     "even = [c for c in tied if (c & 1) == 1]", "ties to the odd code"),
    ("fp8.py", "return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)",
     "return sign * (1.0 + m / 8.0) * 2.0 ** (e - 8)", "exponent bias 8"),
    ("fp8.py",
     "    prod = np.minimum(np.maximum(prod, np.float32(-MAX)), np.float32(MAX))\n",
     "", "no saturation before rounding"),
    ("fp8.py", "    prod = x32 * np.asarray(inv_scale, dtype=np.float32)",
     "    prod = x32 * np.asarray(inv_scale, dtype=np.float32).T",
     "per-head scales on the wrong axis"),
    ("prefix_cache.py",
     'data = struct.pack("<QQ", parent & MASK64, salt & MASK64)',
     'data = struct.pack("<QQ", 0, salt & MASK64)', "key ignores the parent"),
    ("prefix_cache.py",
     "if e is None or e.parent != parent or e.tokens != toks:\n            return None",
     "if e is None:\n            return None", "collision taken as a hit"),
    ("prefix_cache.py", "for e in reversed(entries):", "for e in entries:",
     "chains stamped head first"),
    ("prefix_cache.py", "for _, k in cands[:max(0, n)]:",
     "for _, k in cands[::-1][:max(0, n)]:", "most recent evicted first"),
    ("allocator.py", "ids = [self.free.popleft() for _ in range(n)]",
     "ids = [self.free.pop() for _ in range(n)]", "LIFO instead of FIFO"),
    ("allocator.py", "            if self.rc[b] == 0:\n                self.free.append(b)",
     "            if self.rc[b] == 0:\n                self.free.appendleft(b)",
     "freed block to the head of the queue"),
    ("allocator.py", "        self.rc[new] = 1\n        self.rc[b] -= 1",
     "        self.rc[new] = 1", "copy-on-write keeps the old reference"),
    ("allocator.py", "            if off == 0:", "            if off == 1:",
     "new block at the wrong offset"),
]


def _mutated_tree(tmp, fname, old, new):
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(tmp, "oracle"),
                    ignore=shutil.ignore_patterns("__pycache__"))
    os.makedirs(os.path.join(tmp, "tests"))
    for f in ("conftest.py",) + PIN_FILES:
        shutil.copy(os.path.join(ROOT, "tests", f),
                    os.path.join(tmp, "tests", f))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"),
                    os.path.join(tmp, "tests", "golden"))
    path = os.path.join(tmp, "oracle", fname)
    src = open(path).read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    with open(path, "w") as f:
        f.write(src.replace(old, new))


def _run_pins(tmp):
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
    return subprocess.run(
        [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
         "-m", "not gpu"] + [os.path.join("tests", f) for f in PIN_FILES],
        cwd=tmp, env=env, capture_output=True, text=True, timeout=600)


def test_unmutated_copy_passes(tmp_path):
    _mutated_tree(str(tmp_path), "attention.py", "import numpy as np",
                  "import numpy as np")
    r = _run_pins(str(tmp_path))
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]


@pytest.mark.parametrize("fname,old,new,what", MUTATIONS,
                         ids=[m[3] for m in MUTATIONS])
def test_pins_catch_planted_mistake(tmp_path, fname, old, new, what):
    _mutated_tree(str(tmp_path), fname, old, new)
    r = _run_pins(str(tmp_path))
    assert r.returncode == 1, (
        f"the pins did not catch: {what}\n" + r.stdout[-2000:])
