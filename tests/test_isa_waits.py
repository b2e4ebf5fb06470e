"""The register-ring kernels wait for their LDS copies with hand-counted
s_waitcnt vmcnt(N) before the workgroup barrier: N counts the vector-memory
instructions a wave issues after the hidden-fragment copies of the chunk it is
about to read. That count holds only while the compiler keeps the issue order
of the source (weight loads, wait, barrier, hidden copies). This test compiles
csrc/gemm_dma.hip for gfx950 on the CPU and checks, in the loop of every
instantiated ring kernel, that

- each hand wait is followed by the barrier before any LDS read;
- walking back from each wait through the loop (cyclically), the N most
  recent vector-memory instructions hold no LDS copy of the chunk being read,
  and the (N+1)-th is an LDS copy, i.e. the wait covers those copies exactly;
- no full drain (vmcnt(0)) sits inside the loop.

A compiler change that moves a load across the wait, splits a body or drains
the pipeline makes it fail, instead of leaving the parity tests to catch an
early LDS read on the GPU.

It also checks the main loop of every LDS-fed kernel (gemm_argmax_dma):
each barrier comes right after a hand wait with no LDS copy between them
(a copy sunk below the wait would make it too weak), and two things that
keep results right but cost speed are absent: a scalar reload of a kernel
argument, and a full drain (vmcnt(0)) right before an LDS read."""

import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "speculative_decoding_argmax_amd"))

VMEM = re.compile(r"^\s*(buffer_load_\w+|global_load_\w+)\b(.*)$")
WAIT = re.compile(r"^\s*s_waitcnt\b.*\bvmcnt\((\d+)\)")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    import build as b
    try:
        hipcc = b.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    if not shutil.which(hipcc) and not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa") / "gemm_dma.s"
    src = os.path.join(ROOT, "speculative_decoding_argmax_amd", "csrc", "gemm_dma.hip")
    cmd = [hipcc, *b.COMMON, *b.DEVICE_FLAGS, "--cuda-device-only", "-S", src, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def kernels(text, stem):
    """{mangled name: body lines} of the kernels whose name starts with stem."""
    out = {}
    for m in re.finditer(rf"^({stem}\w*):", text, re.M):
        name = m.group(1)
        end = text.index(f".Lfunc_end", m.end())
        out[name] = text[m.end():end].split("\n")
    return out


def loop_of(lines):
    """Lines of the kernel's main loop in cyclic execution order: the blocks
    the compiler marks as inside the first loop header, starting at the
    header; blocks placed before it (the latch the back edge jumps to) come
    last."""
    hdr = next(i for i, l in enumerate(lines) if "Loop Header" in l)
    tag = "BB" + lines[hdr].split(":")[0].strip().lstrip(".L").split("BB", 1)[1]
    starts = [i for i, l in enumerate(lines) if re.match(r"^\.LBB\d+_\d+:", l)] + [len(lines)]
    after, before = [], []
    for a, b in zip(starts, starts[1:]):
        head = lines[a]
        if a == hdr or f"Header={tag} " in head:
            (after if a >= hdr else before).append(lines[a:b])
    return [l for blk in after + before for l in blk]


def check_ring_loop(loop):
    events = []  # ("mem", is_lds) | ("wait", n) | ("bar",) | ("ds",)
    for l in loop:
        m = VMEM.match(l)
        if m:
            events.append(("mem", " lds" in m.group(2) or "_lds" in m.group(1)))
            continue
        w = WAIT.match(l)
        if w:
            events.append(("wait", int(w.group(1))))
        elif re.match(r"^\s*s_barrier\b", l):
            events.append(("bar",))
        elif re.match(r"^\s*ds_read", l):
            events.append(("ds",))
    mem = [i for i, e in enumerate(events) if e[0] == "mem"]
    waits = [i for i, e in enumerate(events) if e[0] == "wait"]
    assert mem and waits, "no loads or waits found in the loop"
    assert all(events[i][1] > 0 for i in waits), "full drain (vmcnt(0)) inside the ring loop"
    hand = [i for i in waits if any(e[0] == "bar" for e in events[i + 1:i + 3])]
    assert hand, "no wait directly before a barrier"
    for i in hand:
        n = events[i][1]
        # the barrier comes before any LDS read after the wait
        nxt = next(e[0] for e in events[i + 1:] if e[0] in ("bar", "ds"))
        assert nxt == "bar", "an LDS read precedes the barrier"
        # walk back cyclically over the loop's vector-memory instructions
        before = [k for k in mem if k < i][::-1] + [k for k in mem if k > i][::-1]
        assert len(before) > n, (n, len(before))
        assert events[before[n]][1], f"vmcnt({n}): the {n + 1}-th older load is no LDS copy"
    return len(hand)


def test_ring_kernel_waits_cover_their_copies(asm):
    rings = kernels(asm, "_ZN3mtp16gemm_argmax_ring")
    assert len(rings) >= 2, sorted(rings)  # tiled and row-major forms
    for name, lines in rings.items():
        n_hand = check_ring_loop(loop_of(lines))
        depth = int(re.match(r"_ZN3mtp16gemm_argmax_ringILi\d+ELi\d+ELi\d+ELi(\d+)E", name).group(1))
        # one hand wait per ring slot: the loop is unrolled by the ring depth
        assert n_hand == depth, (name, n_hand, depth)


def test_checker_flags_a_moved_copy(asm):
    """The check itself: moving the hidden copies of a body above its weight
    loads (so the wait no longer covers them) must fail it."""
    rings = kernels(asm, "_ZN3mtp16gemm_argmax_ring")
    loop = loop_of(next(iter(rings.values())))
    lds_lines = [i for i, l in enumerate(loop) if VMEM.match(l) and " lds" in l]
    first_load = next(i for i, l in enumerate(loop) if VMEM.match(l) and " lds" not in l)
    # hoist every LDS copy to the start of the loop
    moved = [loop[0]] + [loop[i] for i in lds_lines] + \
            [l for i, l in enumerate(loop[1:], 1) if i not in set(lds_lines)]
    assert first_load > 0
    with pytest.raises(AssertionError):
        check_ring_loop(moved)


def test_checker_flags_loads_sunk_below_the_wait(asm):
    """The check itself, on the reordering a compiler could plausibly make:
    the weight loads issued just before a hand wait moved below it. The wait
    then counts older instructions, no longer this chunk's copies."""
    for lines in kernels(asm, "_ZN3mtp16gemm_argmax_ring").values():
        loop = loop_of(lines)
        w = next(i for i, l in enumerate(loop) if WAIT.match(l))
        loads = [i for i in range(w) if VMEM.match(loop[i]) and " lds" not in loop[i]]
        block = [i for i in loads if i > loads[0]] + [loads[0]]
        moved = [l for i, l in enumerate(loop) if i not in set(block) and i != w]
        at = moved.index(next(l for l in loop[w + 1:] if re.match(r"^\s*s_barrier\b", l)))
        moved[at:at] = [loop[w]]                       # wait just before the barrier
        moved[at + 2:at + 2] = [loop[i] for i in sorted(block)]  # loads after it
        with pytest.raises(AssertionError):
            check_ring_loop(moved)


def mfma_loop(lines):
    """Lines of the loop that holds the kernel's first MFMA: every block the
    compiler marks as that loop's header or as inside it."""
    starts = []
    for i, l in enumerate(lines):
        m = re.match(r"^(\.LBB\d+_\d+|; %bb\.\d+):(.*)$", l)
        if m:
            name = m.group(1)
            name = "BB" + name.split("BB", 1)[1] if name.startswith(".LBB") else name
            inside = re.search(r"in Loop: Header=(\w+)", m.group(2))
            starts.append((i, name if "Loop Header" in m.group(2) else
                           (inside.group(1) if inside else None)))
    starts.append((len(lines), None))
    first = next(i for i, l in enumerate(lines) if "v_mfma" in l)
    hdr = starts[max(j for j, b in enumerate(starts[:-1]) if b[0] <= first)][1]
    assert hdr is not None, "the first MFMA is in no loop"
    return [l for j, b in enumerate(starts[:-1]) if b[1] == hdr
            for l in lines[b[0]:starts[j + 1][0]]]


def check_dma_loop(loop):
    """Inside the copy/MFMA loop of the LDS-fed kernel: no scalar reload of a
    kernel argument, and no full drain of the copies in flight right before
    an LDS read (the waits before the reads are the hand-counted ones)."""
    ins = [l.strip() for l in loop
           if l.strip() and not l.strip().startswith(";") and not re.match(r"^[.\w%]+:", l.strip())]
    for i, l in enumerate(ins):
        assert not l.startswith("s_load"), f"scalar load inside the loop: {l}"
        if re.match(r"s_waitcnt\b.*\bvmcnt\(0\)", l):
            nxt = next((x for x in ins[i + 1:i + 4] if not x.startswith("s_nop")), "")
            assert not nxt.startswith("ds_read"), f"vmcnt(0) right before {nxt}"


def test_dma_kernel_loops_keep_copies_in_flight(asm):
    """Every LDS-fed matrix-core kernel (gemm_argmax_dma) keeps its copies in
    flight across the LDS reads of its main loop. A larger kernel argument
    once pushed the compiler, at the scalar-register limit, into reloading an
    argument inside the loop and draining every copy before an LDS read: 10%
    slower, with correct results."""
    dmas = kernels(asm, "_ZN3mtp15gemm_argmax_dma")
    assert len(dmas) >= 20, len(dmas)
    for name, lines in dmas.items():
        try:
            check_dma_loop(mfma_loop(lines))
        except AssertionError as e:
            raise AssertionError(f"{name}: {e}") from None


def check_dma_barriers(loop, nbuf):
    """Inside the loop of the LDS-fed kernel: one barrier per LDS slot (the
    loop is unrolled by the slot count), each right after a hand wait
    vmcnt(n > 0), with no LDS copy between that wait and the barrier. The
    copies of a body are issued after its barrier and must stay ahead of the
    next body's wait: a copy sunk below that wait would no longer count as
    younger, and the wait would then let the oldest copies of the chunk
    about to be read still be in flight. (The barrier's compiler fence stops
    a copy from sinking further.)"""
    ev = []
    for l in loop:
        s = l.strip()
        m = VMEM.match(l)
        if m:
            ev.append(("copy" if (" lds" in m.group(2) or "_lds" in m.group(1)) else "load",))
            continue
        w = WAIT.match(l)
        if w:
            ev.append(("wait", int(w.group(1))))
        elif re.match(r"s_barrier\b", s):
            ev.append(("bar",))
        elif s and not s.startswith(";") and not re.match(r"^[.\w%]+:", s):
            ev.append(("op",))
    bars = [i for i, e in enumerate(ev) if e[0] == "bar"]
    assert len(bars) == nbuf, f"{len(bars)} barriers in a loop of {nbuf} slots"
    for b in bars:
        hand = next((j for j in range(b - 1, max(b - 24, -1), -1)
                     if ev[j][0] == "wait" and ev[j][1] > 0), None)
        assert hand is not None, "no hand wait right before a barrier"
        assert all(e[0] != "copy" for e in ev[hand + 1:b]), "an LDS copy between a hand wait and its barrier"


def test_dma_kernel_waits_precede_their_barriers(asm):
    """Every LDS-fed kernel keeps each body's copies ahead of the next body's
    hand wait (check_dma_barriers)."""
    dmas = kernels(asm, "_ZN3mtp15gemm_argmax_dma")
    for name, lines in dmas.items():
        nbuf = int(re.match(r"_ZN3mtp15gemm_argmax_dmaILi\d+ELi\d+ELi\d+ELi(\d+)E", name).group(1))
        try:
            check_dma_barriers(mfma_loop(lines), nbuf)
        except AssertionError as e:
            raise AssertionError(f"{name}: {e}") from None


def test_dma_barrier_checker_flags_a_sunk_copy(asm):
    """The check itself: an LDS copy moved between a hand wait and its
    barrier must fail it."""
    name, lines = next(iter(kernels(asm, "_ZN3mtp15gemm_argmax_dma").items()))
    nbuf = int(re.match(r"_ZN3mtp15gemm_argmax_dmaILi\d+ELi\d+ELi\d+ELi(\d+)E", name).group(1))
    loop = mfma_loop(lines)
    check_dma_barriers(loop, nbuf)
    copy = next(l for l in loop if VMEM.match(l) and "lds" in l)
    k = next(i for i, l in enumerate(loop) if re.match(r"^\s*s_barrier\b", l))
    with pytest.raises(AssertionError):
        check_dma_barriers(loop[:k] + [copy] + loop[k:], nbuf)


def test_dma_checker_flags_a_drain_before_an_lds_read(asm):
    """The check itself: a full drain inserted before the first LDS read of
    a loop, or a scalar load inside it, must fail it."""
    lines = next(iter(kernels(asm, "_ZN3mtp15gemm_argmax_dma").values()))
    loop = mfma_loop(lines)
    check_dma_loop(loop)
    k = next(i for i, l in enumerate(loop) if l.strip().startswith("ds_read"))
    with pytest.raises(AssertionError):
        check_dma_loop(loop[:k] + ["\ts_waitcnt vmcnt(0)"] + loop[k:])
    with pytest.raises(AssertionError):
        check_dma_loop(loop[:k] + ["\ts_load_dwordx4 s[40:43], s[0:1], 0x20"] + loop[k:])
