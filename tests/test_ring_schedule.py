"""The LDS weight ring of the streaming GEMMs, checked on the CPU.

The streaming gate_up and down kernels fetch weight slabs into a ring of S
LDS slots with direct-to-LDS loads and find out that a slab has arrived by a
fixed `s_waitcnt vmcnt(N)`: "at most N of my vector loads are still in
flight".  That is only right if (a) the issue/wait schedule lands every
slab before it is read and never refills a slot that is still being read,
under in-order retirement of vector loads, and (b) the compiled loop issues
exactly the loads the schedule counts between its waits.  (a) is checked by
simulating the schedule of both ring forms (per-wave tokens, and tokens
shared by a workgroup of four waves) for every slot count, token-group
count and tile count the library builds; planted mistakes show the
simulation catches what it should.  (b) is checked on the device assembly
the build keeps (`_build/expert_gemm-gfx950.s`): in every ring loop of every
kernel instance, the number of vector-memory instructions between
consecutive hand-written waits equals the count the wait assumes, and
`_build/*.resources.json` (the compiler's resource-usage remarks) shows no
kernel with counted waits uses scratch memory, whose reloads would be
vector loads the count does not know of.
"""
import json
import os
import re
from dataclasses import dataclass, field

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "_build")
SHARE_WAVES = 4


class Violation(AssertionError):
    pass


@dataclass
class Wave:
    """One wave's vector-memory queue (in-order retirement) and LDS reads."""
    queue: list = field(default_factory=list)   # (kind, slab, slot, q) in issue order
    reading: set = field(default_factory=set)   # ring slots with LDS reads not yet returned

    def issue(self, load):
        self.queue.append(load)

    def wait_vm(self, n, landed):
        """s_waitcnt vmcnt(n): retire all but the n youngest loads."""
        keep = self.queue[len(self.queue) - n:] if n else []
        for ld in self.queue[:len(self.queue) - len(keep)]:
            landed.add(ld)
        self.queue = keep

    def drain_lds(self):
        self.reading.clear()


def simulate_private(S, NG, NW, nsl, young=None, drain=True):
    """contract_dma: per-wave weight ring, tokens into registers one slab ahead.

    Step j: drain LDS reads; issue slab j+S-1 (clamped to the last slab)
    into slot (j+S-1)%S as 2 NW loads and the tokens of slab j+1 as 2 NG
    loads; vmcnt(P); read slot j%S and the tokens of slab j.  Returns the
    number of slabs each wait has landed ahead of the one it guards."""
    P = 2 * NW + 2 * NG
    young = P if young is None else young
    w = Wave()
    landed = set()
    content = {}          # slot -> slab most recently issued into it

    def dma(slab, slot):
        if slot in w.reading:
            raise Violation(f"slot {slot} refilled while read (step slab {slab})")
        content[slot] = slab
        for t in range(NW):
            for i in range(2):
                w.issue(("W", slab, slot, (t, i)))

    def tload(slab):
        for h in range(2):
            for g in range(NG):
                w.issue(("T", slab, None, (h, g)))

    for j in range(S - 1):
        dma(min(j, nsl - 1), j)
    tload(0)
    ahead = []
    for j in range(nsl):
        if drain:
            w.drain_lds()
        dma(min(j + S - 1, nsl - 1), (j + S - 1) % S)
        tload(min(j + 1, nsl - 1))
        w.wait_vm(young, landed)
        slot = j % S
        need = [("W", j, slot, (t, i)) for t in range(NW) for i in range(2)]
        if content.get(slot) != j or not all(ld in landed for ld in need):
            raise Violation(f"S={S} NG={NG} NW={NW} nsl={nsl}: slab {j} read before it landed")
        if not all(("T", j, None, (h, g)) in landed for h in range(2) for g in range(NG)):
            raise Violation(f"tokens of slab {j} read before they landed")
        # slabs beyond j whose loads are all retired: the slack of this wait
        k = 0
        while j + k + 1 < nsl and all(("W", j + k + 1, (j + k + 1) % S, (t, i)) in landed
                                      for t in range(NW) for i in range(2)):
            k += 1
        ahead.append(k)
        w.reading.add(slot)
    w.wait_vm(0, landed)
    return ahead


def simulate_shared(S, NG, NW, nsl, young=None, drain=True):
    """contract_shared: four waves, per-wave weight rings and one token ring.

    The 2 NG token loads of a slab are dealt round the waves (wave w issues
    loads (w + 4 c) % 2NG, c < ceil(2NG/4)).  Iteration j: each wave waits
    vmcnt((S-2) P) (+ lgkmcnt(0) when drain), all meet at a barrier, then
    each issues slab j+S-1 into slot (j+S-1)%S and reads slot j%S."""
    kti = (2 * NG + SHARE_WAVES - 1) // SHARE_WAVES
    P = 2 * NW + kti
    young = (S - 2) * P if young is None else young
    waves = [Wave() for _ in range(SHARE_WAVES)]
    landed = set()
    reading_tok = [set() for _ in range(SHARE_WAVES)]

    def issue(wv, slab, slot):
        w = waves[wv]
        if slot in w.reading:
            raise Violation(f"weight slot {slot} refilled while read")
        if any(slot in r for r in reading_tok):
            raise Violation(f"token slot {slot} refilled while some wave reads it")
        for t in range(NW):
            for i in range(2):
                w.issue(("W", slab, slot, (wv, t, i)))
        for c in range(kti):
            q = (wv + c * SHARE_WAVES) % (2 * NG)
            w.issue(("X", slab, slot, q))

    for wv in range(SHARE_WAVES):
        for j in range(S - 1):
            issue(wv, min(j, nsl - 1), j)
    for j in range(nsl):
        for wv, w in enumerate(waves):          # wait, then the barrier
            w.wait_vm(young, landed)
            if drain:
                w.drain_lds()
                reading_tok[wv].clear()
        for wv in range(SHARE_WAVES):           # after the barrier
            issue(wv, min(j + S - 1, nsl - 1), (j + S - 1) % S)
        slot = j % S
        for wv, w in enumerate(waves):
            if not all(("W", j, slot, (wv, t, i)) in landed for t in range(NW) for i in range(2)):
                raise Violation(f"S={S} NG={NG}: weight slab {j} read before it landed")
            if not all(any(ld[0] == "X" and ld[1] == j and ld[2] == slot and ld[3] == q
                           for ld in landed) for q in range(2 * NG)):
                raise Violation(f"S={S} NG={NG}: token slab {j} read before it landed")
            w.reading.add(slot)
            reading_tok[wv].add(slot)
    for w in waves:
        w.wait_vm(0, landed)


# every (S, NG, NW) the library instantiates: S in 2..4 slots; NG token
# groups 1, 2 or 4 (blocks of 16..64 rows, leading groups only); NW = 2
# for gate_up (gate + up tile) and 1 or 2 for down
INSTANCES = [(S, NG, NW) for S in (2, 3, 4) for NG in (1, 2, 4) for NW in (1, 2)]


@pytest.mark.parametrize("S,NG,NW", INSTANCES)
def test_private_ring_schedule_lands_every_slab(S, NG, NW):
    for nsl in range(1, 13):
        ahead = simulate_private(S, NG, NW, nsl)
        # the wait that guards slab j has also landed slabs j+1 .. j+S-2
        assert all(a >= min(S - 2, nsl - 1 - j) for j, a in enumerate(ahead))


@pytest.mark.parametrize("S,NG,NW", INSTANCES)
def test_shared_ring_schedule_lands_every_slab(S, NG, NW):
    for nsl in range(1, 13):
        simulate_shared(S, NG, NW, nsl)


@pytest.mark.parametrize("S", [2, 3, 4])
def test_schedule_model_catches_planted_mistakes(S):
    # one load too many left in flight: the two-slot ring reads an unlanded slab
    # (with more slots the extra slack absorbs it: the margin is S - 2 slabs)
    if S == 2:
        with pytest.raises(Violation):
            simulate_private(S, 1, 2, 8, young=2 * 2 + 2 * 1 + 2 * 1 + 1)
    with pytest.raises(Violation):  # a wait that counts a whole extra slab
        simulate_private(S, 1, 2, 8, young=(2 * 2 + 2) * (S - 1) + 2 + 1)
    with pytest.raises(Violation):  # no LDS drain before a slot is refilled
        simulate_private(S, 1, 2, 8, drain=False)
    with pytest.raises(Violation):  # the shared ring waiting for one slab too few
        simulate_shared(S, 2, 2, 8, young=(S - 1) * (2 * 2 + 1))
    with pytest.raises(Violation):  # no drain before the barrier
        simulate_shared(S, 2, 2, 8, drain=False)


# ------------------------------------------------------- compiled loops

_VMEM = re.compile(r"^\s*(global|buffer|flat|scratch)_(load|store|atomic)\w*\s")
_NAME = re.compile(r"^(_ZN7moelora12_GLOBAL__N_1(\d+)(k_gate_up|k_down)I\w+):")


def _template_args(mangled):
    """(TG, ..., S, SH) of a k_gate_up / k_down instance, from its mangled name."""
    return [int(v) for v in re.findall(r"L[ib](\d+)E", mangled)]


def _functions(text):
    cur, lines = None, []
    for line in text.splitlines():
        m = _NAME.match(line)
        if m or (cur and re.match(r"^\.Lfunc_end", line)):
            if cur:
                yield cur, lines
            cur, lines = (m.group(1), m.group(3)) if m else None, []
            continue
        if cur:
            lines.append(line)


def _loops(lines):
    """Bodies of the innermost loops, in execution order: the compiler marks
    each loop's header block and every other block of the loop ("in Loop:
    Header=..."); the body is the header block and the member blocks after
    it, then the member blocks laid out before it (a latch placed ahead of
    the header)."""
    blocks = []   # [label, annotation, lines]
    for l in lines:
        m = re.match(r"^(\.LBB\w+):\s*(;.*)?$", l)
        if m:
            blocks.append([m.group(1), m.group(2) or "", []])
        elif blocks and not blocks[-1][2] and re.match(r"^\s*;", l):
            # a nested loop's header carries its notes on comment lines of
            # their own ("Parent Loop ...", then "=>  This Inner Loop Header")
            blocks[-1][1] += " " + l.strip()
        elif blocks:
            blocks[-1][2].append(l)
    for i, (label, note, _) in enumerate(blocks):
        if not re.search(r"=>\s*This Inner Loop Header", note):
            continue
        tag = "Header=" + label.lstrip(".")
        member = lambda b: b[0] == label or re.search(re.escape(tag) + r"\b", b[1])
        after = [b for b in blocks[i:] if member(b)]
        before = [b for b in blocks[:i] if member(b)]
        body = []
        for b in after + before:
            body.append(f"{b[0]}:")
            body.extend(b[2])
        yield body


def _hand_waits(body):
    """(index, vmcnt) of the hand-written waits: an s_waitcnt with a vmcnt
    field between two empty inline-asm compiler barriers."""
    out = []
    for i, l in enumerate(body):
        m = re.match(r"^\s*s_waitcnt\s+vmcnt\((\d+)\)", l)
        if m and i >= 2 and ";;#ASMEND" in body[i - 1] and i + 1 < len(body) \
                and ";;#ASMSTART" in body[i + 1]:
            out.append((i, int(m.group(1))))
    return out


ASM = os.path.join(BUILD, "expert_gemm-gfx950.s")


@pytest.mark.skipif(not os.path.exists(ASM), reason="device assembly not built "
                    "(python lora_expert_gemm_amd/build.py)")
def test_compiled_ring_loops_issue_what_their_waits_count():
    text = open(ASM).read()
    seen = {2: 0, 3: 0, 4: 0, "w8": 0}
    for (name, kind), lines in _functions(text):
        args = _template_args(name)   # ..., [R2,] S, SH, W8
        S, SH, W8 = args[-3], bool(args[-2]), bool(args[-1])
        if S == 0:
            assert not any(_hand_waits(b) for b in _loops(lines)), name
            continue
        TG = args[0]
        R2 = kind == "k_down" and bool(args[-4])
        NW = 2 if kind == "k_gate_up" or R2 else 1
        ngs = {1, 2, TG} & {1, 2, 4}
        ngs = {g for g in ngs if g <= TG}
        # token loads per slab: 2 NG (bf16, 64-wide slabs) or 4 NG (E4M3,
        # 128-wide slabs), dealt round the four waves when shared
        tok = {g: (4 if W8 else 2) * g for g in ngs}
        if SH:
            per = {2 * NW + (tok[g] + SHARE_WAVES - 1) // SHARE_WAVES for g in ngs}
        else:
            per = {2 * NW + tok[g] for g in ngs}
        found = set()
        for body in _loops(lines):
            waits = _hand_waits(body)
            if not waits:
                continue
            idx = [i for i, _ in waits]
            vm = [sum(1 for l in body[a:b] if _VMEM.match(l))
                  for a, b in zip(idx, idx[1:] + [len(body) + idx[0]])]
            # cyclic: the window after the last wait wraps to the loop head
            vm[-1] = sum(1 for l in body[idx[-1]:] if _VMEM.match(l)) + \
                sum(1 for l in body[:idx[0]] if _VMEM.match(l))
            assert len(set(vm)) == 1, f"{name}: uneven loads between waits {vm}"
            p = vm[0]
            assert p in per, f"{name}: {p} loads per step, expected one of {per}"
            want = (S - 2) * p if SH else p
            assert all(n == want for _, n in waits), \
                f"{name}: waits {[n for _, n in waits]} for {p} loads per step (S={S})"
            found.add(p)
        assert found, f"{name}: no ring loop with hand-written waits found"
        seen[S] += 1
        seen["w8"] += W8
    assert all(seen.values()), seen


@pytest.mark.skipif(not os.path.exists(os.path.join(BUILD, "expert_gemm.hip.resources.json")),
                    reason="resource remarks not built")
def test_kernels_with_counted_waits_use_no_scratch():
    for src in ("expert_gemm.hip", "tiled_gemm.hip"):
        res = json.load(open(os.path.join(BUILD, src + ".resources.json")))
        assert res, src
        for name, r in res.items():
            assert r["ScratchSize"] == 0 and r["VGPRs Spill"] == 0 and r["SGPRs Spill"] == 0, name
