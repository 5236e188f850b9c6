"""The page loops of the streaming kernels keep their next page's requests in
flight: compiled to gfx950 assembly (on the CPU, with the library's own
flags), the loop that streams the pages holds no `s_waitcnt vmcnt(0)`.

A page loop requests page p+1's operands at the top of page p and waits for
page p's with a partial count.  The compiler can only count the requests in
flight where every path through the loop issued the same ones: a branch
around a request, a page skipped by a branch, or operands copied from the
next page's registers into the current page's turn the wait into vmcnt(0),
which waits for the next page's requests too and leaves the pipeline one
memory round trip per page.  Each case names a kernel instance and the
product that marks its page loop (the outermost loop holding the most of
them)."""
import os
import re
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from rank_compressed_paged_amd import build  # noqa: E402

CASES = [
    # (source, mangled kernel name, product in the page loop)
    ("generic.hip", "_ZN6starkv20generic_split_kernelILb0ELi8ELb1ELb0EEEvNS_7GenArgsE",
     "v_mfma_f32_16x16x16_f16"),
    ("generic.hip", "_ZN6starkv20generic_split_kernelILb1ELi8ELb1ELb0EEEvNS_7GenArgsE",
     "v_mfma_f32_16x16x16_f16"),
    ("generic.hip", "_ZN6starkv22generic_prefill_kernelILb0EEEvNS_7GenArgsEi",
     "v_mfma_f32_16x16x16_f16"),
    ("generic.hip", "_ZN6starkv22generic_prefill_kernelILb1EEEvNS_7GenArgsEi",
     "v_mfma_f32_16x16x16_f16"),
]
DECODE_SPLIT = re.compile(r"^(_ZN6starkv19decode_split_kernelILi32ELi64ELi512ELi16ELi2ELb0ELi1ELb[01]\S*):")


def _assembly(src, outdir):
    out = os.path.join(outdir, src + ".s")
    cmd = [build.hipcc(), *build.compile_flags(), "-x", "hip", "--cuda-device-only", "-S",
           os.path.join(build.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read().splitlines()


def _function(lines, name):
    start = next(i for i, l in enumerate(lines) if l.startswith(name + ":"))
    end = next(i for i in range(start, len(lines)) if lines[i].startswith(".Lfunc_end"))
    return lines[start:end]


def _page_loop(body, product):
    """Lines of the outermost loop holding the most `product` instructions.
    A loop's blocks are the ones the compiler's block comments place in it
    (header `=>This ... Loop Header: Depth=1`, body `Header=BBn Depth=1`,
    nested headers `Parent Loop BBn Depth=1`)."""
    loops, cur = {}, None
    for l in body:
        m = re.match(r"^(\.LBB\w+|; %bb\.\d+):\s*(.*)$", l)
        if m:
            label, note = m.group(1), m.group(2)
            if "Loop Header: Depth=1" in note:
                cur = label[2:]  # .LBB7_22 -> BB7_22
            else:
                h = re.search(r"(?:Header=|Parent Loop )(BB\w+) Depth=1", note)
                cur = h.group(1) if h else (cur if "Depth=2" in note else None)
        if cur:
            loops.setdefault(cur, []).append(l)
    best = max(loops.values(), key=lambda ls: sum(product in x for x in ls), default=None)
    assert best is not None and any(product in x for x in best), "no page loop found"
    return best


@pytest.fixture(scope="module")
def asm():
    if not os.path.exists(build.hipcc()):
        pytest.skip("hipcc not installed")
    d = tempfile.mkdtemp(prefix="starkv_isa_")
    try:
        yield {src: _assembly(src, d) for src in ("generic.hip", "decode.hip")}
    finally:
        shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("src,name,product", CASES, ids=[c[1][8:40] for c in CASES])
def test_generic_page_loops_wait_for_their_own_page(asm, src, name, product):
    loop = _page_loop(_function(asm[src], name), product)
    waits = [l.strip() for l in loop if re.search(r"s_waitcnt.*vmcnt\(0\)", l)]
    partial = [l for l in loop if re.search(r"s_waitcnt.*vmcnt\([1-9]", l)]
    assert not waits, waits
    assert partial, "the page loop waits for no request at all"


def test_tuned_decode_split_page_loop_waits_for_its_own_page(asm):
    names = [DECODE_SPLIT.match(l).group(1) for l in asm["decode.hip"] if DECODE_SPLIT.match(l)]
    assert names
    for name in names:
        loop = _page_loop(_function(asm["decode.hip"], name), "v_mfma")
        assert not [l for l in loop if re.search(r"s_waitcnt.*vmcnt\(0\)", l)], name
