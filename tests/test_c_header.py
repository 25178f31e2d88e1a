"""include/vc.h is a plain C header: a strict C99 program (gcc -std=c99 -pedantic -Werror)
includes it, links libvc.so and calls the entry points that need no GPU (version, status
strings, workspace sizes, argument validation)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "bit_attention_video_online_amd")

PROG = r"""
#include <stdio.h>
#include <string.h>
#include "vc.h"
int main(void) {
  int bad = 0;
  if (vc_abi_version() != VC_ABI_VERSION) bad |= 1;
  if (vc_max_clusters() != 8192) bad |= 2;
  if (strncmp(vc_status_string(VC_E_SHAPE), "VC_E_SHAPE", 10) != 0) bad |= 4;
  /* the quantiser's workspace at the video workload's size: 22 bytes per block element + the rest */
  if (vc_quantize_workspace_bytes(1, 40, 70400, 128, 128) < (size_t)22 * 40 * 550 * 128) bad |= 8;
  if (vc_quantize_workspace_bytes(1, 40, 70400, 128, 64) != 0) bad |= 16;
  if (vc_cluster_workspace_bytes(1, 1, 256, 128, 257) != 0) bad |= 32;
  /* validation runs before any device work: a null input is VC_E_NULLPTR */
  if (vc_cluster(NULL, 1, 1, 256, 128, 8, 1, 1, NULL, NULL, NULL, NULL, 0, NULL) != VC_E_NULLPTR) bad |= 64;
  printf("%d\n", bad);
  return bad;
}
"""


def test_header_is_strict_c99_and_links():
    if not os.path.exists(os.path.join(LIBDIR, "libvc.so")):
        pytest.skip("libvc.so not built")
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    import tempfile
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "abi.c"), os.path.join(d, "abi")
        open(src, "w").write(PROG)
        cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(ROOT, "include"), src,
               "-L", LIBDIR, "-lvc", "-Wl,-rpath," + LIBDIR, "-o", exe]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
        assert r.returncode == 0 and r.stdout.strip() == "0", (r.returncode, r.stdout, r.stderr)
