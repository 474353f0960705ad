"""The Stage-1 split-K hand-off, checked on the CPU (no GPU needed).

Every Stage-1 kernel splits its input rows over several blocks per output
panel; each block writes its partial sums to the workspace and takes a ticket,
and the block that draws the last ticket adds the partials in fixed split
order.  The hand-off uses no cache-wide maintenance.  Its correctness rests on
two things this file checks:

1. The gfx950 code the compiler generates keeps the sequence: partials
   stored with agent-coherent stores (sc1, written through to the level all
   XCDs share), every storing thread waiting for its stores (s_waitcnt
   vmcnt(0)) and the block synchronising (s_barrier) before the ticket
   atomic; after the atomic, a wait and a block barrier before any
   agent-coherent (sc1) load of the partials; and no buffer_wbl2 or
   buffer_inv anywhere in the kernel.  A compiler or flag change that moved
   a load above the ticket, dropped a coherence bit or the wait fails here.
2. A model of the protocol (blocks as interleaved event sequences, stores
   becoming visible at arbitrary later times unless waited for): over many
   random schedules the last-ticket block always reads every fresh partial,
   exactly one block reduces, the ticket returns to 0 for the next call, and
   the result is bit-identical whatever the arrival order.  Without the wait
   the model finds schedules that read a stale partial (negative control).

The opt-in fused Stage-2 kernel joins its two phases with a grid barrier of
per-block epoch flags and bounded waits; a model of that protocol checks the
same properties (no block passes before every block's stores are visible,
flags consistent across launches, including launches whose blocks give up),
with the same kind of negative control, and its generated code is checked for
the arrival sequence the protocol assumes (phase-A stores complete, first
W_down batch still in flight, block barrier, then the flag).  Its k_s is
published by the block
that draws the last completion ticket, so a give-up (-1) cannot be overwritten
by a late k_s; a model checks that too, with the single-writer race it
replaces as negative control.
"""
import os
import random
import re
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "free_ffn_activation_amd", "csrc")

# (source, kernel-name substring) of every kernel with the split-K hand-off
HANDOFF_KERNELS = [("stage1.hip", "stage1_kernel"), ("stage1_batch.hip", "stage1_batch_kernel"),
                   ("stage1_w16.hip", "stage1_w16_kernel")]


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


def _device_asm(src: str, tmp_path) -> str:
    from free_ffn_activation_amd import build_lib
    flags = [f for f in build_lib.FLAGS if f not in ("-shared", "-fPIC")]
    out = os.path.join(str(tmp_path), src + ".s")
    cmd = [_hipcc(), *flags, "--cuda-device-only", "-S", "-I", os.path.join(ROOT, "include"),
           os.path.join(CSRC, src), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    with open(out) as fh:
        return fh.read()


def _kernel_bodies(asm: str, name_part: str):
    """{symbol: [instruction lines]} for the kernels whose symbol contains name_part."""
    bodies, cur, name = {}, None, None
    for line in asm.splitlines():
        m = re.match(r"^(_Z\S+):", line)
        if m:
            name = m.group(1)
            cur = [] if name_part in name else None
            if cur is not None:
                bodies[name] = cur
            continue
        if cur is None:
            continue
        ins = line.split(";")[0].strip()
        if not ins or ins.startswith(".") or ins.endswith(":"):
            continue
        cur.append(ins)
        if ins.startswith("s_endpgm"):
            cur = None
    return bodies


def _is_sc1_store(i):
    return i.startswith("global_store") and re.search(r"\bsc1\b", i) is not None


def _is_sc1_load(i):
    return i.startswith("global_load") and re.search(r"\bsc1\b", i) is not None


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
@pytest.mark.parametrize("src,kernel", HANDOFF_KERNELS)
def test_handoff_sequence_in_generated_code(src, kernel, tmp_path):
    bodies = _kernel_bodies(_device_asm(src, tmp_path), kernel)
    assert bodies, f"no {kernel} in the generated code of {src}"
    for sym, ins in bodies.items():
        assert not any(i.startswith(("buffer_wbl2", "buffer_inv")) for i in ins), \
            f"{sym}: cache-wide maintenance in the kernel"
        tickets = [k for k, i in enumerate(ins) if i.startswith("global_atomic_add")]
        assert len(tickets) == 1, f"{sym}: expected one ticket atomic, found {len(tickets)}"
        t = tickets[0]
        assert "sc0" in ins[t].split(), f"{sym}: the ticket atomic must return its value"
        stores = [k for k in range(t) if _is_sc1_store(ins[k])]
        assert stores, f"{sym}: no agent-coherent partial store before the ticket"
        # after the last agent-coherent store: a full vmcnt wait, then a barrier, then the ticket
        between = ins[stores[-1] + 1:t]
        w = [k for k, i in enumerate(between) if re.match(r"s_waitcnt\s+vmcnt\(0\)", i)]
        b = [k for k, i in enumerate(between) if i.startswith("s_barrier")]
        assert w and b and w[0] < b[-1], f"{sym}: stores not waited for and synchronised before the ticket"
        # no plain store of partial data may follow the coherent ones before the ticket
        assert not any(i.startswith("global_store") for i in between), f"{sym}: store between wait and ticket"
        # no agent-coherent load before the ticket; after it a wait and a barrier precede the first one
        assert not any(_is_sc1_load(i) for i in ins[:t]), f"{sym}: partial load above the ticket"
        loads = [k for k in range(t + 1, len(ins)) if _is_sc1_load(ins[k])]
        assert loads, f"{sym}: no agent-coherent partial load after the ticket"
        after = ins[t + 1:loads[0]]
        w2 = [k for k, i in enumerate(after) if re.match(r"s_waitcnt\s+vmcnt\(0\)", i)]
        b2 = [k for k, i in enumerate(after) if i.startswith("s_barrier")]
        assert w2 and b2 and w2[0] < b2[0], f"{sym}: partials read before the ticket's result was shared"


# ---------------------------------------------------------------- protocol model
def _simulate(splits, partials, rng, with_wait=True, ticket0=0):
    """One call of the hand-off for one panel under a random schedule.

    Block b: store its partial (issued), [wait until visible], take a ticket;
    the block drawing splits-1 reads all partials (a partial not yet visible
    reads as the stale value NaN) and adds them in split order, then resets
    the ticket.  A store becomes visible at any later step of the schedule.
    Returns (sum, reducers, final ticket, stale reads)."""
    memory = [np.float32(np.nan)] * splits        # stale contents from an earlier call
    pending = {}                                   # block -> value issued, not yet visible
    state = {b: "store" for b in range(splits)}
    ticket = ticket0
    reducers, total, stale = [], None, 0
    while True:
        moves = []
        for b, st in state.items():
            if st == "store":
                moves.append(("store", b))
            elif st == "ticket" and (not with_wait or b not in pending):
                moves.append(("ticket", b))
        moves += [("visible", b) for b in pending]
        if not moves:
            break
        kind, b = rng.choice(moves)
        if kind == "store":
            pending[b] = partials[b]
            state[b] = "ticket"
        elif kind == "visible":
            memory[b] = pending.pop(b)
        else:
            prev = ticket
            ticket += 1
            state[b] = "done"
            if prev == splits - 1:
                reducers.append(b)
                acc = np.float32(0.0)
                for k in range(splits):               # fixed split order
                    v = memory[k]
                    stale += int(np.isnan(v))
                    acc = np.float32(acc + v)
                total = acc
                ticket = 0                            # ready for the next call
    for b, v in pending.items():
        memory[b] = v
    return total, reducers, ticket, stale


def test_ticket_protocol_model():
    rng = random.Random(7)
    for splits in (2, 3, 8, 16):
        partials = [np.float32(v) for v in np.random.default_rng(splits).standard_normal(splits)]
        ref = np.float32(0.0)
        for v in partials:
            ref = np.float32(ref + v)
        for _ in range(400):
            total, reducers, ticket, stale = _simulate(splits, partials, rng)
            assert len(reducers) == 1 and ticket == 0 and stale == 0
            assert np.float32(total).view(np.uint32) == ref.view(np.uint32)   # bit-identical


def test_ticket_protocol_model_needs_the_wait():
    """Negative control: without waiting for its stores before the ticket, a
    block can hand over before its partial is visible."""
    rng = random.Random(11)
    partials = [np.float32(v) for v in range(1, 9)]
    stale = sum(_simulate(8, partials, rng, with_wait=False)[3] for _ in range(400))
    assert stale > 0


# ---------------------------------------------------------------- fused Stage-2 grid barrier
def _barrier_call(flags, rng, wait_limit, allow_early_flag=False):
    """One launch of the fused Stage-2 kernel's barrier over G blocks, under a
    random schedule.  Block b: read its own flag (epoch = flag + 1); phase A
    (publishes its s values); store flags[b] = epoch — only after its phase-A
    stores are complete unless allow_early_flag (the mistake the model must
    catch); then poll every flag until all have reached the epoch, or give up
    after wait_limit of its own polling steps.  Returns (blocks that passed
    with some s value not yet visible, blocks that gave up)."""
    G = len(flags)
    epoch = {}
    published = {b: False for b in range(G)}  # phase-A stores visible to every block
    state = {b: "read" for b in range(G)}
    polls = {b: 0 for b in range(G)}
    stale, gave_up = 0, 0
    while any(st != "done" for st in state.values()):
        b = rng.choice([k for k, st in state.items() if st != "done"])
        st = state[b]
        if st == "read":
            epoch[b] = flags[b] + 1
            state[b] = "phaseA"
        elif st == "phaseA":
            state[b] = "flag" if allow_early_flag else "ack"
            if not allow_early_flag:
                published[b] = True      # waited for (vmcnt) before the flag
        elif st == "ack":
            state[b] = "flag"
        elif st == "flag":
            flags[b] = epoch[b]
            state[b] = "poll"
            if allow_early_flag and rng.random() < 0.5:
                published[b] = True      # may become visible later
        elif st == "poll":
            if all(flags[k] - epoch[b] >= 0 for k in range(G)):
                stale += int(not all(published.values()))
                state[b] = "done"
            else:
                polls[b] += 1
                if polls[b] > wait_limit:
                    gave_up += 1
                    state[b] = "done"
        for k in range(G):               # late visibility of early flags' data
            if state[k] in ("poll", "done") and not published[k] and rng.random() < 0.3:
                published[k] = True
    return stale, gave_up


def test_grid_barrier_protocol_model():
    """Epoch flags: no block passes before every block's phase-A stores are
    visible; the flags stay equal between launches (fresh workspace: all 0);
    a launch whose blocks give up (wait bound 0) leaves them equal too, so the
    next launch with the normal bound is correct."""
    rng = random.Random(3)
    for G in (2, 5, 16):
        flags = [0] * G
        for call in range(60):
            limit = 0 if call % 7 == 3 else 10 ** 9
            stale, gave_up = _barrier_call(flags, rng, limit)
            assert stale == 0
            assert len(set(flags)) == 1 and flags[0] == call + 1
            if limit > 0:
                assert gave_up == 0


def test_grid_barrier_protocol_model_needs_the_wait():
    """Negative control: a flag stored before the block's own stores are
    complete lets some block pass while an s value is not yet visible."""
    rng = random.Random(5)
    flags = [0] * 8
    stale = sum(_barrier_call(flags, rng, 10 ** 9, allow_early_flag=True)[0] for _ in range(200))
    assert stale > 0


# ---------------------------------------------------------------- fused Stage-2 k_s publication
def _publish_count(G, gave_up, rng, ticketed=True, done0=0):
    """Who writes mask_count in one launch of the fused Stage-2 kernel.

    ticketed: every block, at its end, adds 1 (+ 1 << 16 if it gave up) to a
    completion counter; the block drawing the last ticket writes k_s or -1
    and resets the counter.  Otherwise (the mistake the model must catch)
    block 0 writes k_s during its first phase and a block that gives up writes
    -1 at its wait, both at arbitrary points of the schedule.
    Returns (final mask_count, final counter)."""
    ks = 1234
    mask_count = 77                              # stale value of an earlier launch
    done = done0
    if ticketed:
        for b in rng.sample(range(G), G):        # order in which blocks finish
            mine = 1 + (0x10000 if b in gave_up else 0)
            prev = done
            done += mine
            if (prev & 0xFFFF) == G - 1:
                done = 0
                mask_count = -1 if ((prev + mine) >> 16) else ks
        return mask_count, done
    writes = [("ks", 0)] + [("gu", b) for b in gave_up]
    rng.shuffle(writes)
    for kind, _ in writes:
        mask_count = ks if kind == "ks" else -1
    return mask_count, done


def test_fused_count_publication_model():
    """k_s is -1 exactly when some block of the launch gave up, whatever the
    finishing order, and the counter is 0 again for the next launch."""
    rng = random.Random(13)
    for G in (1, 2, 7, 256):
        for _ in range(300):
            gave_up = set(b for b in range(G) if rng.random() < 0.05)
            mc, done = _publish_count(G, gave_up, rng)
            assert mc == (-1 if gave_up else 1234) and done == 0


def test_fused_count_publication_needs_one_writer():
    """Negative control: with block 0 writing k_s and give-ups writing -1
    independently, some schedules end with k_s although a block gave up."""
    rng = random.Random(17)
    lost = sum(_publish_count(8, {3, 5}, rng, ticketed=False)[0] != -1 for _ in range(200))
    assert lost > 0


# ---------------------------------------------------------------- fused Stage-2 barrier arrival
def _kernel_lines(asm: str, name_part: str):
    """{symbol: [instruction or label lines]} (labels kept, comments dropped)."""
    bodies, cur = {}, None
    for line in asm.splitlines():
        m = re.match(r"^(_Z\S+):", line)
        if m:
            cur = [] if name_part in m.group(1) else None
            if cur is not None:
                bodies[m.group(1)] = cur
            continue
        if cur is None:
            continue
        ins = line.split(";")[0].strip()
        if not ins or ins.startswith("."):
            if ins.startswith(".LBB"):
                cur.append(ins)
            continue
        cur.append(ins)
        if ins.startswith("s_endpgm"):
            cur = None
    return bodies


def _down_unroll() -> int:
    with open(os.path.join(CSRC, "prox_internal.h")) as fh:
        return int(re.search(r"constexpr int kDownUnroll = (\d+);", fh.read()).group(1))


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_fused_barrier_arrival_in_generated_code(tmp_path):
    """The fused Stage-2 kernel arrives at its grid barrier only after its
    phase-A stores are complete, without waiting for the first W_down batch:
    the last kDownUnroll vector-memory instructions before its
    s_waitcnt vmcnt(kDownUnroll) are those loads, in straight-line code (no
    label between them and the wait), and the wait is followed by the block
    barrier and then the device-coherent flag store.  A store moved into the
    window, or a branch, would let a block publish its flag early."""
    k = _down_unroll()
    bodies = _kernel_lines(_device_asm("stage2_fused.hip", tmp_path), "stage2_fused_kernel")
    assert len(bodies) == 2, f"expected the bf16 and fp32 kernels, found {list(bodies)}"
    for sym, ins in bodies.items():
        waits = [i for i, s in enumerate(ins) if s == f"s_waitcnt vmcnt({k})"
                 and any(t.startswith("s_barrier") for t in ins[i + 1:i + 3])]
        arrivals = []
        for w in waits:
            after = ins[w + 1:w + 20]
            b = next(j for j, t in enumerate(after) if t.startswith("s_barrier"))
            st = [j for j, t in enumerate(after) if t.startswith("global_store") and re.search(r"\bsc1\b", t)]
            if st and st[0] > b:
                arrivals.append(w)
        assert len(arrivals) == 1, f"{sym}: expected one barrier arrival, found {len(arrivals)}"
        w = arrivals[0]
        vmem = [i for i in range(w) if ins[i].startswith(("global_", "buffer_", "flat_", "scratch_"))]
        last = vmem[-k:]
        assert all(ins[i].startswith("global_load_dwordx4") for i in last), \
            f"{sym}: the {k} operations before the arrival wait are not all W_down loads"
        assert not any(t.startswith(".LBB") or t.startswith("s_cbranch") or t.startswith("s_branch")
                       for t in ins[last[0]:w]), f"{sym}: control flow between the W_down loads and the wait"
        assert not any(ins[i].startswith(("global_store", "global_atomic", "buffer_store", "scratch_store"))
                       for i in range(last[0], w)), f"{sym}: a store inside the window"
