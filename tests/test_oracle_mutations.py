"""Pin strength: plausible mistakes planted in a copy of the oracle must make
its pins fail.

Each case copies ``oracle/``, the oracle pin tests and their golden files into
a temporary folder, changes one expression of the copy (a dropped bit, a
shifted field, an off-by-one, a reversed tie-break, a flipped sign, a wrong
index), and runs the pin tests that should notice it against the copy in a
fresh interpreter.  They must fail (pytest exit status 1); a mutant that
survives means a pin is missing.  The real oracle is never modified.
"""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

# (name, oracle file, original text, planted text, pin test files)
MUTANTS = [
    ("raw byte drops a mantissa bit", "fields.py",
     "mantissa = (b & 0x7F).astype(np.uint8)", "mantissa = (b & 0x3F).astype(np.uint8)",
     ["test_oracle_codebook.py", "test_oracle_stream.py"]),
    ("exponent taken one bit too high", "fields.py",
     "exponent = ((b >> 7) & 0xFF).astype(np.uint8)", "exponent = ((b >> 8) & 0xFF).astype(np.uint8)",
     ["test_oracle_codebook.py", "test_oracle_stream.py"]),
    ("package-merge keeps one item too many", "codebook.py",
     "chosen = current[: 2 * m - 2]", "chosen = current[: 2 * m - 1]",
     ["test_oracle_codebook.py"]),
    ("package-merge runs one round too few", "codebook.py",
     "for _ in range(max_len - 1):", "for _ in range(max_len - 2):",
     ["test_oracle_codebook.py"]),
    ("canonical codes skip a value between lengths", "codebook.py",
     "code = (code + count[l - 1]) << 1 if l > 1 else 0", "code = (code + count[l - 1] + 1) << 1 if l > 1 else 0",
     ["test_oracle_codebook.py"]),
    ("packer writes bits LSB-first", "stream.py",
     "words[pos >> 5] |= 1 << (31 - (pos & 31))", "words[pos >> 5] |= 1 << (pos & 31)",
     ["test_oracle_stream.py"]),
    ("vectorised packer places codes one bit off", "stream.py",
     "v = c << (np.uint64(64) - r - l.astype(np.uint64))", "v = c << (np.uint64(63) - r - l.astype(np.uint64))",
     ["test_oracle_stream.py", "test_oracle_blob.py"]),
    ("chunk offset skips a code starting on the boundary", "stream.py",
     'idx = np.searchsorted(starts, chunk_first[live], side="left")',
     'idx = np.searchsorted(starts, chunk_first[live], side="right")',
     ["test_oracle_stream.py"]),
    ("block offsets count codes starting on the boundary", "stream.py",
     'out[:n_blocks] = np.searchsorted(starts, block_first, side="left")',
     'out[:n_blocks] = np.searchsorted(starts, block_first, side="right")',
     ["test_oracle_stream.py"]),
    ("5-bit offset fields bit-reversed", "stream.py",
     "g = 5 * np.arange(off.size, dtype=np.int64) + k", "g = 5 * np.arange(off.size, dtype=np.int64) + (4 - k)",
     ["test_oracle_stream.py", "test_oracle_blob.py"]),
    ("entropy bound drops a raw bit", "blob.py",
     "return n * (8.0 + cb.entropy_bits(hist)) / 8.0", "return n * (7.0 + cb.entropy_bits(hist)) / 8.0",
     ["test_oracle_blob.py"]),
    ("rANS frequencies: larger symbol first on tied remainders", "ans.py",
     "order = sorted(present, key=lambda s: (-(h[s] * m % total), s))",
     "order = sorted(present, key=lambda s: (-(h[s] * m % total), -s))",
     ["test_oracle_ans.py"]),
    ("rANS frequencies: take back from the larger symbol on ties", "ans.py",
     "s = max(present, key=lambda t: (f[t], -t))", "s = max(present, key=lambda t: (f[t], t))",
     ["test_oracle_ans.py"]),
    ("rANS renormalises one bit early", "ans.py",
     "if x >= fs << (32 - PROB_BITS):", "if x >= fs << (31 - PROB_BITS):",
     ["test_oracle_ans.py"]),
    ("rANS decoder adds the cumulative frequency", "ans.py",
     "x = int(f[s]) * (x // M) + slot - int(c[s])", "x = int(f[s]) * (x // M) + slot + int(c[s])",
     ["test_oracle_ans.py"]),
    ("padded tails filled with zeros", "padded.py",
     "ones = (np.uint64(1) << gl.astype(np.uint64)) - np.uint64(1)", "ones = np.zeros(gl.shape, dtype=np.uint64)",
     ["test_oracle_padded.py"]),
    ("panel order takes rows from the wrong lane bits", "panel.py",
     "r = r0 + l % 32", "r = r0 + l // 2",
     ["test_oracle_panel.py"]),
    ("GEMM reference reverses K", "gemm.py",
     "return w @ x", "return w @ x[::-1]",
     ["test_oracle_gemm.py"]),
    ("merge puts the sign one bit low", "fields.py",
     "return ((sign << 15) | (e << 7) | mantissa).astype(np.uint16)",
     "return ((sign << 14) | (e << 7) | mantissa).astype(np.uint16)",
     ["test_oracle_codebook.py", "test_oracle_stream.py"]),
    ("Huffman depth counts one level too many", "codebook.py",
     "heapq.heappush(items, (a[0] + b[0], 1, serial, max(a[3], b[3]) + 1))",
     "heapq.heappush(items, (a[0] + b[0], 1, serial, max(a[3], b[3]) + 2))",
     ["test_oracle_codebook.py"]),
    ("Huffman depth takes the shallower subtree", "codebook.py",
     "heapq.heappush(items, (a[0] + b[0], 1, serial, max(a[3], b[3]) + 1))",
     "heapq.heappush(items, (a[0] + b[0], 1, serial, min(a[3], b[3]) + 1))",
     ["test_oracle_codebook.py"]),
    ("Huffman depth of one symbol is zero", "codebook.py",
     "return 1 if items else 0", "return 0",
     ["test_oracle_codebook.py"]),
    ("automatic chunk size tries 32 bytes first", "blob.py",
     "AUTO_CHUNK_ORDER = (16, 32, 8, 4)", "AUTO_CHUNK_ORDER = (32, 16, 8, 4)",
     ["test_oracle_blob.py"]),
    ("automatic chunk size compares against 2.5%", "blob.py",
     "AUTO_SIZE_TARGET = 1.02", "AUTO_SIZE_TARGET = 1.025",
     ["test_oracle_blob.py"]),
    ("closed-form size forgets the guard words", "blob.py",
     "return (HEADER_BYTES + (n_chunks * chunk_bytes + 16) +", "return (HEADER_BYTES + (n_chunks * chunk_bytes) +",
     ["test_oracle_blob.py"]),
    ("entropy in nats", "codebook.py",
     "return float(-(p * np.log2(p)).sum())", "return float(-(p * np.log(p)).sum())",
     ["test_oracle_codebook.py"]),
    ("canonical decode accepts a window equal to the limit", "codebook.py",
     'if window24 < tables["limit"][l]:', 'if window24 <= tables["limit"][l]:',
     ["test_oracle_codebook.py", "test_oracle_stream.py"]),
    ("chunk decoder starts from the next chunk's offset", "stream.py",
     "pos = i * bits + off[:n_chunks]", "pos = i * bits + off[1: n_chunks + 1]",
     ["test_oracle_stream.py"]),
    ("rANS cumulative frequencies shifted by one symbol", "ans.py",
     "c[1:] = np.cumsum(f)[:-1]", "c[1:] = np.cumsum(f)[1:]",
     ["test_oracle_ans.py"]),
    ("rANS lanes interleaved in ascending order", "ans.py",
     "for l in range(lanes - 1, -1, -1):", "for l in range(lanes):",
     ["test_oracle_ans.py"]),
    ("panel items column slices first", "panel.py",
     "for p in range(rows // PANEL_ROWS):\n        for c0 in range(0, cols, panel_k):",
     "for c0 in range(0, cols, panel_k):\n        for p in range(rows // PANEL_ROWS):",
     ["test_oracle_panel.py"]),
    ("padded decoder drops a code ending on the chunk end", "padded.py",
     "if pos + l > end:", "if pos + l >= end:",
     ["test_oracle_padded.py"]),
    ("padded chunk refuses a code ending on its last bit", "padded.py",
     'last = int(np.searchsorted(flat_end, flat_start[first] + bits, side="right"))',
     'last = int(np.searchsorted(flat_end, flat_start[first] + bits, side="left"))',
     ["test_oracle_padded.py"]),
    ("an extra block when the chunks fill whole blocks", "stream.py",
     "blocks = -(-used // lanes)", "blocks = used // lanes + 1",
     ["test_oracle_stream.py", "test_oracle_blob.py"]),
    ("canonical limit one code short", "codebook.py",
     "limit[l] = (first[l] + count[l]) << (MAX_LEN - l)", "limit[l] = (first[l] + count[l] - 1) << (MAX_LEN - l)",
     ["test_oracle_codebook.py", "test_oracle_stream.py"]),
    ("panel item table records the block count for the chunk count", "panel.py",
     "table.append((chunk_base, block_base, bits_q, 0))", "table.append((block_base, block_base, bits_q, 0))",
     ["test_oracle_panel.py"]),
    ("panel block offsets count from the item, not the matrix", "panel.py",
     'outs.append(elem_base + np.searchsorted(starts, first, side="left"))',
     'outs.append(np.searchsorted(starts, first, side="left"))',
     ["test_oracle_panel.py"]),
    ("coded size leaves out the chunk offsets", "blob.py",
     'for nm in ("words", "offsets", "blockout", "raw", "panels", "counts"))',
     'for nm in ("words", "blockout", "raw", "panels", "counts"))',
     ["test_oracle_blob.py", "test_oracle_stream.py"]),
    ("rANS frequencies without the floor of one", "ans.py",
     "f[s] = max(1, h[s] * m // total)", "f[s] = h[s] * m // total",
     ["test_oracle_ans.py"]),
    ("rANS encoder lanes start one above the lower state bound", "ans.py",
     "x = [L] * lanes", "x = [L + 1] * lanes",
     ["test_oracle_ans.py"]),
    ("vectorised rANS encoder renormalises only above the bound", "ans.py",
     "emit = live & (x >= (fs << np.uint64(32 - PROB_BITS)))", "emit = live & (x > (fs << np.uint64(32 - PROB_BITS)))",
     ["test_oracle_ans.py"]),
    ("vectorised rANS encoder keeps a step's words in ascending lane order", "ans.py",
     "out.append((x[emit] & np.uint64(0xFFFF))[::-1])", "out.append(x[emit] & np.uint64(0xFFFF))",
     ["test_oracle_ans.py"]),
    ("panel chunk counts take a code ending a chunk for one starting there", "panel.py",
     "np.bincount(np.asarray(starts, dtype=np.int64) // (8 * chunk_bytes), minlength=chunks_q)",
     "np.bincount((np.asarray(starts, dtype=np.int64) + 1) // (8 * chunk_bytes), minlength=chunks_q)",
     ["test_oracle_panel.py"]),
    ("coded size leaves out the chunk counts", "blob.py",
     'for nm in ("words", "offsets", "blockout", "raw", "panels", "counts"))',
     'for nm in ("words", "offsets", "blockout", "raw", "panels"))',
     ["test_oracle_panel.py"]),
    ("panel sub-tiles eight columns wide", "panel.py",
     "c = c0 + SUBTILE_K * t + 8 * (l // 32) + j", "c = c0 + 8 * t + 8 * (l // 32) + j",
     ["test_oracle_panel.py"]),
    ("bf16 widened to float32 one bit short", "gemm.py",
     "<< np.uint32(16)", "<< np.uint32(15)",
     ["test_oracle_gemm.py"]),
    ("package-merge breaks leaf ties by the larger symbol", "codebook.py",
     "order = sorted(range(m), key=lambda i: (int(hist[used[i]]), used[i]))",
     "order = sorted(range(m), key=lambda i: (int(hist[used[i]]), -used[i]))",
     ["test_oracle_codebook.py"]),
    ("package-merge puts packages before leaves of equal weight", "codebook.py",
     "key=lambda it: (it[0], it[1], it[2]))", "key=lambda it: (it[0], -it[1], it[2]))",
     ["test_oracle_codebook.py"]),
    ("canonical codes of one length in decreasing symbol order", "codebook.py",
     "    for s in range(256):\n        l = int(lengths[s])\n        if l > 0:\n            codes[s] = next_code[l]",
     "    for s in range(255, -1, -1):\n        l = int(lengths[s])\n        if l > 0:\n            codes[s] = next_code[l]",
     ["test_oracle_codebook.py"]),
    ('code starts shifted by one code', 'stream.py',
     'np.cumsum(l[:-1], out=starts[1:])',
     'np.cumsum(l[1:], out=starts[1:])',
     ['test_oracle_stream.py']),
    ('block offsets section one entry short', 'blob.py',
     '"blockout": 4 * (enc["n_blocks"] + 1),',
     '"blockout": 4 * enc["n_blocks"],',
     ['test_oracle_blob.py']),
    ("padded chunks start their codes one bit in", "padded.py",
     "starts[first:last] = chunk * bits + (flat_start[first:last] - flat_start[first])",
     "starts[first:last] = chunk * bits + 1 + (flat_start[first:last] - flat_start[first])",
     ["test_oracle_padded.py"]),
]


def sandbox(tmp_path, files):
    """tmp_path/oracle (a copy) and tmp_path/tests (conftest, golden, files)."""
    ignore = shutil.ignore_patterns("__pycache__", "*.pyc")
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle", ignore=ignore)
    tests = tmp_path / "tests"
    shutil.copytree(os.path.join(HERE, "golden"), tests / "golden", ignore=ignore)
    shutil.copy(os.path.join(HERE, "conftest.py"), tests / "conftest.py")
    for f in files:
        shutil.copy(os.path.join(HERE, f), tests / f)
    return tests


def run_pins(tmp_path, tests, files):
    # the copy first, then the repository for the package (seeded generators)
    env = {**os.environ, "PYTHONPATH": os.pathsep.join([str(tmp_path), ROOT]), "PYTHONDONTWRITEBYTECODE": "1"}
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                           *files], cwd=tests, env=env, capture_output=True, text=True, timeout=600)


def test_unmutated_copy_passes(tmp_path):
    files = ["test_oracle_gemm.py", "test_oracle_panel.py"]
    r = run_pins(tmp_path, sandbox(tmp_path, files), files)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, mutant):
    name, fname, old, new, files = mutant
    tests = sandbox(tmp_path, files)
    path = tmp_path / "oracle" / fname
    src = path.read_text()
    assert src.count(old) == 1, f"{name}: the original text must occur exactly once in oracle/{fname}"
    path.write_text(src.replace(old, new))
    r = run_pins(tmp_path, tests, files)
    assert r.returncode == 1, f"{name}: the pins did not fail (exit {r.returncode})\n" + (r.stdout + r.stderr)[-3000:]
