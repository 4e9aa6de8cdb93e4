"""The streaming kernels' speed rests on a few properties of their machine
code, and the compiler can lose them silently after an innocent source change
(a store sunk past a branch drops its nontemporal flag; a load sunk into a
branch makes the wave wait before issuing the next).  These tests compile the
kernel source for gfx950 to assembly and check, in every instantiation of the
three main kernels:

  - every 16-byte global load and store is nontemporal (`nt`): the state
    stream, and the gather pass's output;
  - the entry pass issues its input and state loads before its first wait;
  - the owner pass issues all its payload-slot loads, its input load and its
    state load before its first wait;
  - the gather pass issues every chunk's loads before its first store.

No GPU is needed: hipcc cross-compiles."""
import os
import re
import subprocess

import pytest

from error_compensated_bit_amd import build as eb

HIPCC = "/opt/rocm/bin/hipcc"
ENTRY = re.compile(r"k_quant_feedbackILi\d+ELi\d+ELi\d+ELi\d+E")
OWNER = re.compile(r"k_owner_reduce_requantILi\d+ELi\d+ELi\d+ELi\d+ELi\d+ELi(\d+)E")
GATHER = re.compile(r"k_dequant_gatherILi\d+ELi\d+ELi\d+ELi(\d+)E")


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not installed")
    out = tmp_path_factory.mktemp("asm") / "echo_kernels.s"
    flags = [f for f in eb.hipcc_flags() if f not in ("-shared", "-fPIC")]
    cmd = [HIPCC] + flags + ["--cuda-device-only", "-S", "-o", str(out),
                             os.path.join(eb.CSRC, "echo_kernels.hip")]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    funcs, name, body = {}, None, []
    for line in open(out):
        m = re.match(r"^(_ZN4echo\w+):", line)
        if m:
            name, body = m.group(1), []
            continue
        if name is not None:
            if line.startswith(".Lfunc_end"):
                funcs[name] = body
                name = None
            else:
                body.append(line.strip())
    return funcs


def instructions(body, prefix):
    return [i for i, s in enumerate(body) if s.startswith(prefix)]


def main_kernels(funcs, pattern):
    found = {n: b for n, b in funcs.items() if pattern.search(n) and "_tail" not in n}
    assert found, f"no kernel matches {pattern.pattern}"
    return found


@pytest.mark.parametrize("pattern", [ENTRY, OWNER, GATHER], ids=["entry", "owner", "gather"])
def test_wide_accesses_are_nontemporal(kernels, pattern):
    for name, body in main_kernels(kernels, pattern).items():
        wide = [s for s in body if s.startswith(("global_load_dwordx4", "global_store_dwordx4"))]
        assert wide, name
        bad = [s for s in wide if not re.search(r"\bnt\b", s)]
        assert not bad, f"{name}: 16-byte accesses without nt: {bad}"


def loads_before_first_wait(body):
    first_wait = min(instructions(body, "s_waitcnt vmcnt") + [len(body)])
    return len([i for i in instructions(body, "global_load") if i < first_wait])


def test_entry_loads_precede_the_first_wait(kernels):
    for name, body in main_kernels(kernels, ENTRY).items():
        assert loads_before_first_wait(body) >= 2, name


def test_owner_issues_every_slot_before_the_first_wait(kernels):
    for name, body in main_kernels(kernels, OWNER).items():
        slots = int(OWNER.search(name).group(1))
        # codes and params of every slot, plus the input and the state
        assert loads_before_first_wait(body) >= 2 * slots + 2, name


def test_gather_issues_every_chunk_before_the_first_store(kernels):
    for name, body in main_kernels(kernels, GATHER).items():
        chunks = int(GATHER.search(name).group(1))
        first_store = min(instructions(body, "global_store"))
        loads = [i for i in instructions(body, "global_load") if i < first_store]
        assert len(loads) >= 2 * chunks, name
