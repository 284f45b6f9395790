"""The boundary from plain C, without a GPU: a C99 program that includes include/dsa.h and
links libdsa.so, built with gcc (no HIP headers, no C++), calls the version, status and
workspace queries and a set of invalid calls that must be rejected before any HIP call."""
import os
import shutil
import subprocess

import pytest

import sparse_attention_05_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

C_SOURCE = r"""
#include <stdio.h>
#include <string.h>
#include "dsa.h"

static int failures = 0;
#define EXPECT(cond) do { if (!(cond)) { printf("FAIL line %d: %s\n", __LINE__, #cond); ++failures; } } while (0)

int main(void)
{
    EXPECT(dsa_version() == 105);
    EXPECT(strcmp(dsa_status_string(DSA_OK), "DSA_OK") == 0);
    EXPECT(strcmp(dsa_status_string(DSA_ERR_WORKSPACE_TOO_SMALL), "DSA_ERR_WORKSPACE_TOO_SMALL") == 0);

    /* size queries: full size_t range, zero for invalid sizes */
    EXPECT(dsa_prefill_chunk_rows(131072, 131072) == 4096);
    EXPECT(dsa_prefill_workspace_bytes(131072, 131072, 64, 128, 2048) > ((size_t)1 << 31));
    EXPECT(dsa_prefill_workspace_bytes(0, 10, 64, 128, 16) == 0);
    EXPECT(dsa_topk_workspace_bytes(4, 100, 8) == 0);
    EXPECT(dsa_decode_noalloc_scratch_bytes() == DSA_DECODE_NOALLOC_SCRATCH_BYTES);

    /* rejected before any HIP call: nothing is launched, nothing written */
    float sc[4] = {1.f, 2.f, 3.f, 4.f};
    int32_t idx[4] = {7, 7, 7, 7};
    EXPECT(dsa_topk(sc, 4, -1, 4, 0, 2, idx, NULL, 0, NULL) == DSA_ERR_INVALID_ARGUMENT);
    EXPECT(dsa_topk(sc, 2, 1, 4, 0, 2, idx, NULL, 0, NULL) == DSA_ERR_INVALID_ARGUMENT);
    EXPECT(dsa_topk(sc, 4, 1, 4, 0, 0, idx, NULL, 0, NULL) == DSA_ERR_INVALID_ARGUMENT);
    EXPECT(dsa_topk(NULL, 4, 1, 4, 0, 2, idx, NULL, 0, NULL) == DSA_ERR_INVALID_ARGUMENT);
    EXPECT(dsa_index_scores(NULL, NULL, NULL, NULL, NULL, 1, 1, 64, 0, 1.f, sc, 1, 0, NULL)
           == DSA_ERR_INVALID_ARGUMENT);
    EXPECT(dsa_sparse_mla(NULL, NULL, NULL, 1, 1, 129, 1, 1.f, NULL, NULL, NULL)
           != DSA_OK);
    EXPECT(dsa_window_indices(1, 1, 0, 0, idx, NULL) == DSA_ERR_INVALID_ARGUMENT);
    EXPECT(dsa_decode_noalloc(1, NULL, 1, 1, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 64, 128,
                              16, 1.f, 1.f, NULL, NULL, NULL, NULL) == DSA_ERR_INVALID_ARGUMENT);
    EXPECT(idx[0] == 7 && idx[3] == 7);
    printf(failures ? "c consumer: %d failures\n" : "c consumer ok\n", failures);
    return failures != 0;
}
"""


def test_plain_c_program_links_and_validates(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    if not os.path.exists(dsa.LIB_PATH):
        from sparse_attention_05_amd import build
        build.build()
    src = tmp_path / "consumer.c"
    src.write_text(C_SOURCE)
    exe = tmp_path / "consumer"
    libdir = os.path.dirname(dsa.LIB_PATH)
    cmd = [gcc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), str(src),
           "-L", libdir, "-l:libdsa.so", "-Wl,-rpath," + libdir, "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and "c consumer ok" in r.stdout, r.stdout + r.stderr
