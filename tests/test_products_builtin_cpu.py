"""Every matrix product of the attention kernels is a compiler builtin.

The compiler places the wait states the matrix-core dependency rules ask
for only around instructions it can see; a product written as inline
assembly would need hand-placed waits that any edit or compiler change can
break silently.  This test compiles each kernel file with the library's
flags to gfx950 assembly (no GPU needed) and checks that it holds matrix
products and that none of them sits inside an inline-assembly block.  (The
only inline assembly left in these files is the global->LDS copy, a
memory instruction whose completion the kernels await explicitly.)"""
import concurrent.futures as cf
import os
import re
import subprocess

import pytest

FILES = ["fwd.hip", "fwd_f32.hip", "dq.hip", "dkdv.hip"]


def _asm(src, out):
    from block_diffusion_lm_bdlm_amd import build as lb
    cmd = [lb._hipcc(), "-x", "hip", "-S", "--cuda-device-only", os.path.join(lb.CSRC, src), "-o", out] \
        + lb._flags() + lb.EXTRA.get(src, [])
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read()


@pytest.fixture(scope="module")
def listings(tmp_path_factory):
    d = tmp_path_factory.mktemp("asm")
    with cf.ThreadPoolExecutor(max_workers=len(FILES)) as ex:
        texts = list(ex.map(lambda f: _asm(f, str(d / (f + ".s"))), FILES))
    return dict(zip(FILES, texts))


@pytest.mark.parametrize("src", FILES)
def test_no_inline_assembly_products(listings, src):
    inline, products, inline_products = False, 0, 0
    for ln in listings[src].split("\n"):
        s = ln.strip()
        if s.startswith(";;#ASMSTART"):
            inline = True
        elif s.startswith(";;#ASMEND"):
            inline = False
        elif re.match(r"^v_mfma", s):
            products += 1
            inline_products += inline
    print(f"{src}: {products} matrix products, {inline_products} in inline assembly")
    assert products > 0
    assert inline_products == 0
