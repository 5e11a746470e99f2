"""Every HIP source compiles and the objects link (CPU: hipcc cross-compiles
for gfx950). Builds into a temporary directory, so the in-tree library the
other tests load is left as it is."""
import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

from tiled_attention_forward_attn_amd.build import ARCH, HIPCC, flags_for, sources


@pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC), reason="hipcc not available")
def test_every_source_compiles_and_links(tmp_path):
    def compile_one(src):
        obj = tmp_path / (os.path.basename(src) + ".o")
        r = subprocess.run([HIPCC, *flags_for(src), "-c", src, "-o", str(obj)],
                           capture_output=True, text=True)
        return src, r.returncode, r.stderr[-4000:], str(obj)

    srcs = sources()
    assert srcs
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(compile_one, srcs))
    failed = [(s, err) for s, rc, err, _ in results if rc != 0]
    assert not failed, "\n".join(f"{s}:\n{err}" for s, err in failed)
    lib = tmp_path / "lib.so"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC",
                        *[o for *_, o in results], "-o", str(lib)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
