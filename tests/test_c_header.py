"""The boundary from C: include/gdn.h compiles as strict C99 and as C++, and a C program
linked against the library reaches every declared entry point and gets the documented
results from the calls that need no GPU (version, status strings, workspace sizing, the
crossover query, and argument errors that are reported before anything is enqueued)."""
import os
import shutil
import subprocess

import pytest

from linear_recurrent_attention_gated_amd import gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")

C_PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "gdn.h"

typedef void (*any_fn)(void);

int main(void) {
    /* every entry point the header declares, by address */
    const any_fn fns[] = {
        (any_fn)gdn_prefill_workspace_bytes, (any_fn)gdn_prefill, (any_fn)gdn_prefill_qknorm,
        (any_fn)gdn_prefill_ex, (any_fn)gdn_prefill_sequential_max_tokens,
        (any_fn)gdn_prefill_prepare, (any_fn)gdn_prefill_scan, (any_fn)gdn_prefill_noalloc,
        (any_fn)gdn_decode_step, (any_fn)gdn_decode_step_qknorm, (any_fn)gdn_decode_step_layers,
        (any_fn)gdn_status_string, (any_fn)gdn_abi_version};
    size_t i;
    char buf[64];
    gdn_decode_layer layer;
    for (i = 0; i < sizeof fns / sizeof fns[0]; ++i)
        if (!fns[i]) return 1;
    printf("abi %d %d\n", gdn_abi_version(), GDN_ABI_VERSION);
    printf("ws %lu %lu\n", (unsigned long)gdn_prefill_workspace_bytes(1, 4096, 16, 32, 128, 128, 64, GDN_BF16),
           (unsigned long)gdn_prefill_workspace_bytes(1, 4096, 16, 32, 128, 128, 48, GDN_BF16));
    printf("xover %d\n", gdn_prefill_sequential_max_tokens(1, 16, 32, 128, 128, GDN_BF16));
    /* argument errors, reported before anything is enqueued */
    printf("null %d\n", (int)gdn_prefill(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1, 64, 2, 4,
                                         32, 32, 16, GDN_BF16, NULL, 0, NULL));
    printf("shape %d\n", (int)gdn_decode_step_layers(&layer, 0, 1, 2, 4, 32, 32, GDN_BF16, 0, NULL));
    printf("flags %d\n", (int)gdn_prefill_ex(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1, 64, 2,
                                             4, 32, 32, 16, GDN_BF16, NULL, 0, NULL, 8u));
    strncpy(buf, gdn_status_string(GDN_ERR_ALIAS), sizeof buf - 1);
    buf[sizeof buf - 1] = 0;
    printf("str %s\n", buf);
    return 0;
}
"""


def _compiler(name):
    path = shutil.which(name)
    if path is None:
        pytest.skip(f"{name} not found")
    return path


def test_header_compiles_as_c99_and_cxx(tmp_path):
    src = tmp_path / "h.c"
    src.write_text('#include "gdn.h"\nint gdn_header_check(void) { return GDN_ABI_VERSION; }\n')
    for cc, std in ((_compiler("gcc"), "-std=c99"), (_compiler("g++"), "-std=c++11")):
        lang = ["-x", "c++"] if cc.endswith("++") else []
        r = subprocess.run([cc, std, "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", INCLUDE, *lang,
                            "-c", str(src), "-o", str(tmp_path / "h.o")], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


def test_c_program_links_and_calls_the_library(tmp_path):
    lib = gdn.LIB_PATH
    if not os.path.exists(lib):
        pytest.skip("library not built")
    src = tmp_path / "use_gdn.c"
    src.write_text(C_PROGRAM)
    exe = tmp_path / "use_gdn"
    libdir = os.path.dirname(lib)
    r = subprocess.run([_compiler("gcc"), "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                        "-I", INCLUDE, str(src), "-o", str(exe), lib, "-Wl,-rpath," + libdir],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    out = dict(line.split(" ", 1) for line in r.stdout.strip().splitlines())
    assert out["abi"] == "1 1"
    ws, ws_bad = (int(x) for x in out["ws"].split())
    assert ws == gdn.gdn_prefill_workspace_bytes(1, 4096, 16, 32, 128, 128, 64, 0) and ws > 0
    assert ws_bad == 0   # chunk 48 is not supported
    assert out["xover"] == "42"
    assert out["null"] == "1" and out["shape"] == "2" and out["flags"] == "3"
    assert out["str"] == gdn.gdn_status_string(5)
