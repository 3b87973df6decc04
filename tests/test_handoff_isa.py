"""The split hand-off as the compiler emits it (CPU only: reads the gfx950 assembly of this
library's own decode kernels).

The combine's correctness rests on how the relaxed device-scope accesses are lowered, not on
release/acquire fences: a split's partial stores must write through to the point where every XCD
sees them (the `sc1` cache policy), complete (`s_waitcnt vmcnt(0)`) before the work-group barrier
and the counter atomic, and the merging work-group must read the partials with `sc1` loads, which
do not hit a stale line in its own XCD's L2.  An agent-scope fence would add an L2 writeback
(`buffer_wbl2`) per work-group.  A compiler or flag change that altered any of this would give wrong
or slow combines without a build error, so this test checks every decode kernel instantiation:

- every buffer store (the partial stores) and every buffer load (the merge's loads) carries sc1;
- the split counter is the first 64-bit atomic, with the returned value requested (sc0), and no
  buffer store comes after it; the only other one is the fused decode-loop step's per-sequence
  count (sparse stored-key kernels), taken after it by the merging work-group;
- between the last buffer store and the atomic there is an `s_waitcnt vmcnt(0)` and then an
  `s_barrier`;
- no `buffer_wbl2` or `buffer_inv` (no cache-wide writeback or invalidate).
"""
import re
import shutil
import subprocess

import pytest

from long_context_decoding_amd import build as B

pytestmark = pytest.mark.skipif(not shutil.which(B.hipcc()) and not B.Path(B.hipcc()).exists(),
                                reason="hipcc not available")


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    # both translation units of the kernels (the default-policy and the streaming-policy halves)
    td = tmp_path_factory.mktemp("isa")
    flags = [f for f in B.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    srcs = [B.CSRC / "ffd_kernels.hip", B.CSRC / "ffd_kernels_stream.hip"]
    procs = [subprocess.Popen([B.hipcc(), *flags, "-S", "--offload-device-only", "-o",
                               str(td / (src.name + ".s")), str(src)],
                              stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
             for src in srcs]
    for pr in procs:
        _, err = pr.communicate()
        assert pr.returncode == 0, err[-4000:]
    bodies = {}
    for src in srcs:
        s = (td / (src.name + ".s")).read_text()
        for m in re.finditer(r"^(_Z\w+):\s*(?:;.*)?$", s, re.M):
            end = s.find(".Lfunc_end", m.end())
            bodies[m.group(1)] = [l.strip() for l in s[m.end():end].splitlines()]
    return {n: b for n, b in bodies.items() if "decode_kernel" in n}


def test_all_decode_kernels_found(kernels):
    # T in {64, 128} x G in {1, 2, 4, 8} x {bf16, fp32} x {sparse, dense} stored-key kernels and
    # T x G x BITS in {2, 4} residual-form kernels, each with the default cache policy; the bf16
    # stored-key and residual-form ones also with the streaming policy
    assert len(kernels) == 80, sorted(kernels)


def test_partials_travel_at_device_scope(kernels):
    for name, lines in kernels.items():
        stores = [i for i, l in enumerate(lines) if l.startswith("buffer_store")]
        loads = [i for i, l in enumerate(lines) if l.startswith("buffer_load")]
        assert stores, name
        for i in stores + loads:
            assert re.search(r"\bsc1\b", lines[i]), (name, lines[i])


def template_args(name):
    """(T, G, BF16, SPARSE, BITS, RES, STREAM) of a mangled decode_kernel name."""
    m = re.search(r"ILi(\d+)ELi(\d+)ELb(\d)ELb(\d)ELi(\d)ELb(\d)ELb(\d)EE", name)
    assert m, name
    return tuple(int(x) for x in m.groups())


def test_stores_complete_before_the_counter(kernels):
    for name, lines in kernels.items():
        _, _, _, sparse, _, res, _ = template_args(name)
        atomics = [i for i, l in enumerate(lines) if l.startswith("global_atomic_add_x2")]
        assert len(atomics) == (2 if sparse and not res else 1), \
            (name, [lines[i] for i in atomics])
        a = atomics[0]
        for i in atomics:
            assert re.search(r"\bsc0\b", lines[i]), (name, lines[i])  # returns the old count
        stores = [i for i, l in enumerate(lines) if l.startswith("buffer_store")]
        assert all(i < a for i in stores), name
        seg = lines[stores[-1] + 1:a]
        waits = [k for k, l in enumerate(seg) if re.match(r"s_waitcnt\s+vmcnt\(0\)", l)]
        barriers = [k for k, l in enumerate(seg) if l == "s_barrier"]
        assert waits and barriers and waits[0] < barriers[-1], (name, seg)


def test_no_cache_wide_fences(kernels):
    for name, lines in kernels.items():
        assert not any(l.startswith(("buffer_wbl2", "buffer_inv")) for l in lines), name
