"""Cache policy of the weight streams, checked in the generated gfx950 code (CPU only).

A decode launch over one token reads every kept proxy slice, up/gate run and
W_down row slice exactly once, so those loads carry the non-temporal hint; a
launch over several tokens reads the rows and channels the tokens share once
per token, and there the hint sent every re-read to memory again (measured:
per-token kernels over 8 tokens 144.5 -> 155.9 us per step).  The per-token
kernels therefore take a template flag, chosen from the grid, and this file
checks that the flag does what it says in the code the compiler generates:

* the one-token instantiation of each per-token kernel issues its weight loads
  (16-byte global or buffer loads) with `nt`, at least one full batch of them;
* the multi-token instantiation issues no load with `nt` at all;
* the grouped kernels (each union row or channel read once per launch) keep
  `nt` on their weight streams;
* the 16-bit proxy's Stage 1 keeps cacheable loads: its lanes read a 64-byte
  chunk each with four 16-byte loads, so every load instruction touches each
  128-byte line of the row segment in part, and with the hint every
  instruction fetched the lines again (measured 1.5x slower).

A compiler or source change that drops or misplaces the hint fails here
without a GPU.
"""
import re

import pytest

from test_handoff_cpu import _device_asm, _hipcc


def _kernel_bodies(asm: str, name_part: str):
    """{symbol: [instruction lines]} of every kernel whose symbol contains
    name_part, the whole function (its early-exit blocks may come before the
    main loop in the layout, so the body runs to the function's end label, not
    to the first s_endpgm)."""
    bodies, cur = {}, None
    for line in asm.splitlines():
        m = re.match(r"^(_Z\S+):", line)
        if m:
            cur = [] if name_part in m.group(1) else None
            if cur is not None:
                bodies[m.group(1)] = cur
            continue
        if line.startswith(".Lfunc_end"):
            cur = None
            continue
        if cur is None:
            continue
        ins = line.split(";")[0].strip()
        if ins and not ins.startswith(".") and not ins.endswith(":"):
            cur.append(ins)
    return bodies

# (source, kernel-name substring, least number of 16-byte nt loads in the
# one-token instantiation: one gather batch of the kernel)
PER_TOKEN = [
    ("stage1.hip", "stage1_kernel", 16),       # 16 gather loads per lane
    ("stage2_upgate.hip", "upgate_kernel", 16),  # 8 steps x (up, gate)
    ("stage2_down.hip", "down_kernel", 4),     # the half batch of a wave's last rows
]
CACHEABLE = [("stage1_w16.hip", "stage1_w16_kernel")]
GROUPED = [
    ("stage2_batch.hip", "upgate_batch_kernel"),
    ("stage2_batch.hip", "down_batch_kernel"),
    ("stage1_qt.hip", "stage1_qt_kernel"),
]

_LOAD16 = re.compile(r"^(global_load_dwordx4|buffer_load_dwordx4)\b")


def _nt_loads(body):
    return sum(1 for i in body if _LOAD16.match(i) and re.search(r"\bnt\b", i))


def _nt_flag(symbol: str) -> int:
    """The last bool template argument of a kernel symbol (the kNt flag)."""
    flags = re.findall(r"Lb([01])E", symbol)
    assert flags, symbol
    return int(flags[-1])


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
@pytest.mark.parametrize("src,kernel,least", PER_TOKEN)
def test_per_token_kernels_hint_only_one_token_launches(src, kernel, least, tmp_path):
    bodies = _kernel_bodies(_device_asm(src, tmp_path), kernel)
    assert bodies, f"no {kernel} in {src}"
    seen = {0: 0, 1: 0}
    for sym, body in bodies.items():
        if kernel + "I" not in sym:
            continue  # a kernel whose name only contains this one
        flag = _nt_flag(sym)
        seen[flag] += 1
        n = _nt_loads(body)
        if flag:
            assert n >= least, f"{sym}: {n} non-temporal 16-byte loads, expected at least {least}"
        else:
            assert n == 0, f"{sym}: {n} non-temporal loads in a multi-token instantiation"
    assert seen[0] > 0 and seen[1] > 0, f"{kernel}: instantiations by flag {seen}"


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
@pytest.mark.parametrize("src,kernel", GROUPED)
def test_grouped_kernels_stream_weights_non_temporally(src, kernel, tmp_path):
    bodies = _kernel_bodies(_device_asm(src, tmp_path), kernel)
    assert bodies, f"no {kernel} in {src}"
    for sym, body in bodies.items():
        assert _nt_loads(body) > 0, f"{sym}: no non-temporal weight loads"


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
@pytest.mark.parametrize("src,kernel", CACHEABLE)
def test_partial_line_gathers_stay_cacheable(src, kernel, tmp_path):
    bodies = _kernel_bodies(_device_asm(src, tmp_path), kernel)
    assert bodies, f"no {kernel} in {src}"
    for sym, body in bodies.items():
        assert _nt_loads(body) == 0, f"{sym}: non-temporal loads in a partial-line gather"
