"""The counted memory waits of the pipelined kernels, checked on the compiled code.

The vocabulary, residual and attention kernels stage operands with
buffer->LDS loads that the compiler does not track, and wait for them with
an explicit s_waitcnt vmcnt(W) before each step's barrier: W is the number
of loads a wave issues after the stage that step consumes. That count is
right only while the compiler emits exactly the loads the source issues,
in that order around the waits. This test compiles the kernels for gfx950
with the library's own flags and checks, per kernel instantiation:

* every counted wait (an s_waitcnt vmcnt(W) directly followed by the
  barrier's s_waitcnt lgkmcnt(0) and s_barrier) has the same W;
* after each counted wait, up to the next one or the closing vmcnt(0), the
  wave issues the same number L of vector memory instructions (one stage's
  loads);
* the loads before the first wait, from the first buffer load on, are the
  stages issued ahead: two stages
  (W = L: one stage left open) for the three-buffer kernels, and for the
  direct kernel's ring of P stages exactly W + L, with W = 4 + (P - 2) L.

No GPU is needed: the checks read the gfx950 assembly hipcc writes here.
"""
import os
import re
import shutil
import subprocess

import pytest

from medusa_draft_heads_amd import build as mdbuild

CSRC = os.path.join(os.path.dirname(mdbuild.__file__), "csrc")

VMEM = re.compile(r"^\s*(buffer_load|buffer_store|buffer_atomic|global_|flat_|scratch_)")
# the compiler may merge its own counters into the same instruction
WAIT = re.compile(r"^\s*s_waitcnt\s+vmcnt\((\d+)\)(?:\s+\w+\(\d+\))*\s*$")

# kernel name part -> kind of pipeline
KERNELS = {
    "k_vocab_mfma_narrow": "three",
    "k_vocab_mfma_cert": "three",
    "k_residual_wide": "three",
    "k_attn_mfma": "three_extra",  # loads of the query rows come before the pipeline
    "k_vocab_mfma_direct": "ring",
}


def _asm(src):
    out = os.path.join(mdbuild.BUILD, os.path.basename(src) + ".s")
    os.makedirs(mdbuild.BUILD, exist_ok=True)
    cmd = ([mdbuild.HIPCC] + mdbuild.FLAGS + mdbuild.FILE_FLAGS.get(os.path.basename(src), []) +
           ["--cuda-device-only", "-S", src, "-o", out])
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    with open(out) as f:
        return f.read()


def _functions(text):
    """(symbol, body lines) of every kernel in an assembly listing."""
    funcs = {}
    for m in re.finditer(r"^(_Z\S+):\s*(?:;.*)?$", text, re.M):
        name = m.group(1)
        end = text.find(".Lfunc_end", m.end())
        if end < 0:
            continue
        body = [ln.split(";")[0].rstrip() for ln in text[m.end():end].splitlines()]
        funcs[name] = [ln for ln in body if ln.strip()]
    return funcs


def _counted_waits(lines):
    """Indices of the s_waitcnt vmcnt(W) lines that open a step: the next
    s_barrier follows within a few lines, after the barrier's lgkmcnt(0),
    with no memory instruction or other vmcnt wait in between."""
    out = []
    for i, ln in enumerate(lines):
        m = WAIT.match(ln)
        if not m:
            continue
        seen_lgkm = False
        for k in range(i + 1, min(i + 8, len(lines))):
            t = lines[k].strip()
            if VMEM.match(t) or t.startswith("s_waitcnt vmcnt") or LABEL.match(t) or t.startswith("s_cbranch") \
                    or t.startswith("s_branch"):
                break
            if re.match(r"^s_waitcnt\s+lgkmcnt\(0\)$", t):
                seen_lgkm = True
            if t == "s_barrier":
                if seen_lgkm:
                    out.append((i, int(m.group(1))))
                break
    return out


LABEL = re.compile(r"^(\.LBB\w+):$")
CLOSE = re.compile(r"^\s*s_waitcnt\s+vmcnt\(0\)")


def _successors(lines, labels, i):
    t = lines[i].strip()
    op = t.split()[0] if t else ""
    if op == "s_endpgm":
        return []
    if op == "s_branch":
        return [labels[t.split()[1]]]
    if op.startswith("s_cbranch"):
        return [labels[t.split()[1]], i + 1]
    return [i + 1] if i + 1 < len(lines) else []


def _walk(lines, labels, start, stops, report, counting=True):
    """Vector memory instructions on every path from line start to the first
    line in stops (the counted waits and the closing vmcnt(0) waits), for the
    paths whose stop is in report. With counting False the count starts at
    the path's first buffer load. Paths that end the program without reaching
    a stop are not reported."""
    found, seen, todo = set(), set(), [(start, counting, 0)]
    while todo:
        i, on, n = todo.pop()
        if (i, on, n) in seen:
            continue
        seen.add((i, on, n))
        if i in stops:
            if i in report:
                found.add(n)
            continue
        t = lines[i].strip()
        if not on and t.startswith("buffer_load"):
            on = True
        if on and VMEM.match(t):
            n += 1
        assert n < 1000, "unbounded path"
        for j in _successors(lines, labels, i):
            todo.append((j, on, n))
    return found


def _check(name, kind, lines):
    waits = _counted_waits(lines)
    assert waits, "%s: no counted wait found" % name
    waits = [(i, w) for i, w in waits if w > 0]  # vmcnt(0) before a barrier closes a pipeline
    assert waits, "%s: no counted wait found" % name
    ws = {w for _, w in waits}
    assert len(ws) == 1, "%s: counted waits differ: %s" % (name, sorted(ws))
    W = ws.pop()
    labels = {LABEL.match(ln.strip()).group(1): i for i, ln in enumerate(lines) if LABEL.match(ln.strip())}
    wait_at = {i for i, _ in waits}
    stops = wait_at | {i for i, ln in enumerate(lines) if CLOSE.match(ln)}
    # from each counted wait to the next one (or the closing wait), on every path: one stage's loads
    segs = set()
    for i in sorted(wait_at):
        segs |= _walk(lines, labels, i + 1, stops, stops)
    assert len(segs) == 1, "%s: loads per step differ by path: %s" % (name, sorted(segs))
    L = segs.pop()
    assert L > 0, name
    # ahead of the first wait, from the first buffer load on: the stages issued
    # before the loop (stores and loads before it, such as clearing the bounds,
    # are older than every stage and do not count)
    pro = _walk(lines, labels, 0, stops, wait_at, counting=False)
    assert len(pro) == 1, "%s: loads ahead of the first wait differ by path: %s" % (name, sorted(pro))
    pro = pro.pop()
    if kind == "three":
        assert W == L, "%s: wait leaves %d loads open, a stage is %d" % (name, W, L)
        assert pro == 2 * L, "%s: %d loads ahead of the first wait, two stages are %d" % (name, pro, 2 * L)
    elif kind == "three_extra":
        assert W == L, "%s: wait leaves %d loads open, a stage is %d" % (name, W, L)
        assert pro >= 2 * L, "%s: %d loads ahead of the first wait, two stages are %d" % (name, pro, 2 * L)
    else:
        assert pro == W + L, "%s: %d loads ahead of the first wait, expected W + L = %d" % (name, pro, W + L)
        assert (W - 4) % L == 0 and W >= 4, "%s: W = %d is not 4 + (P - 2) L with L = %d" % (name, W, L)
    return W, L, len(waits)


@pytest.fixture(scope="module")
def listings():
    if not os.path.exists(mdbuild.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc is not installed")
    return {f: _asm(os.path.join(CSRC, f)) for f in ("heads_mfma.hip", "attention.hip")}


def test_counted_waits_match_the_issued_loads(listings):
    seen = {k: 0 for k in KERNELS}
    for text in listings.values():
        for name, lines in _functions(text).items():
            part = next((k for k in KERNELS if k in name), None)
            if part is None:
                continue
            _check(name, KERNELS[part], lines)
            seen[part] += 1
    missing = [k for k, c in seen.items() if c == 0]
    assert not missing, "kernels not found in the listings: %s" % missing


def _one(listings, part, src="heads_mfma.hip", template=""):
    return next((n, l) for n, l in _functions(listings[src]).items() if part in n and template in n)


def test_the_check_rejects_a_dropped_load(listings):
    # a step that issues one load fewer than the wait assumes must fail
    name, lines = _one(listings, "k_residual_wide")
    i0 = _counted_waits(lines)[1][0]
    j = next(i for i in range(i0 + 1, len(lines)) if VMEM.match(lines[i]))
    with pytest.raises(AssertionError, match="loads per step"):
        _check(name, "three", lines[:j] + lines[j + 1:])


def test_the_check_rejects_a_wrong_count(listings):
    # one wait that leaves a load more open than the others must fail
    name, lines = _one(listings, "k_vocab_mfma_cert")
    i0, w = _counted_waits(lines)[2]
    broken = list(lines)
    broken[i0] = broken[i0].replace("vmcnt(%d)" % w, "vmcnt(%d)" % (w + 1))
    with pytest.raises(AssertionError, match="counted waits differ"):
        _check(name, "three", broken)


def test_the_check_rejects_dropped_ring_loads(listings):
    # the direct kernel's tail with its U loads gone (what dropping unused
    # ring loads does) must fail: each tail step then issues only the
    # activation pieces
    name, lines = _one(listings, "k_vocab_mfma_direct", template="ILi2ELi5ELb1ELb1E")
    waits = _counted_waits(lines)
    i0 = waits[-1][0]
    nxt = next((i for i in range(i0 + 1, len(lines)) if CLOSE.match(lines[i])), len(lines))
    drop = [i for i in range(i0 + 1, nxt) if re.match(r"^\s*buffer_load\w*\s+v\[", lines[i])]
    assert len(drop) == 4, drop  # the step's four U fragments (register loads)
    broken = [ln for i, ln in enumerate(lines) if i not in drop]
    with pytest.raises(AssertionError, match="loads per step"):
        _check(name, "ring", broken)
