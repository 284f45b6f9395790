"""Host sanitizer builds (CPU only).

* The oracle (oracle/oracle.c) built with gcc under AddressSanitizer and
  UndefinedBehaviorSanitizer, driven through every entry point on small random inputs,
  ragged shapes and edge cases included (one key, k >= n, padding in index lists).
* The C ABI layer (api.cpp) built with the same sanitizers on its host code only (hipcc with
  -Xarch_host before each -fsanitize=, so device code is untouched), driven through argument
  validation and the workspace-size queries, which never reach the GPU.

Any sanitizer report fails the test (UBSan without recovery, ASan with leak checks off: the
HIP runtime keeps process-lifetime allocations)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

ORACLE_DRIVER = r"""
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include "oracle.h"

static uint32_t rs = 12345u;
static uint32_t rnd(void) { rs = rs * 1664525u + 1013904223u; return rs >> 8; }
static uint8_t code(void) { uint8_t c = (uint8_t)rnd(); return (c & 0x7F) == 0x7F ? 0 : c; }
static uint16_t bf16(void) { return (uint16_t)(0x3F00u | (rnd() & 0x80FFu)); }

int main(void)
{
    const int T = 19, L = 37, H_I = 4, H = 8, k = 7, q_pos0 = L - T;
    uint8_t* q8 = malloc(T * H_I * 128); uint8_t* k8 = malloc(L * 128);
    float* qs = malloc(sizeof(float) * T * H_I); float* w = malloc(sizeof(float) * T * H_I);
    float* ks = malloc(sizeof(float) * L);
    for (int i = 0; i < T * H_I * 128; ++i) q8[i] = code();
    for (int i = 0; i < L * 128; ++i) k8[i] = code();
    for (int i = 0; i < T * H_I; ++i) { qs[i] = 0.01f * (1 + rnd() % 7); w[i] = (float)((int)(rnd() % 9) - 4); }
    for (int i = 0; i < L; ++i) ks[i] = 0.02f * (1 + rnd() % 5);
    int64_t rows[19]; for (int i = 0; i < T; ++i) rows[i] = i;
    double* sc = malloc(sizeof(double) * T * L); double* bd = malloc(sizeof(double) * T * L);
    int bad = 0;
    bad |= ora_index_scores(q8, qs, w, k8, ks, L, H_I, q_pos0, 0.088, rows, T, sc, bd);
    int64_t nv[19]; for (int i = 0; i < T; ++i) nv[i] = q_pos0 + i + 1;
    int32_t* i1 = malloc(4 * T * k); int32_t* i2 = malloc(4 * T * k);
    bad |= ora_topk_sort(sc, L, T, nv, k, i1);
    bad |= ora_topk_select(sc, L, T, nv, k, i2);
    if (memcmp(i1, i2, 4 * T * k)) { printf("selectors differ\n"); bad = 1; }
    int32_t* big = malloc(4 * T * 64);
    bad |= ora_topk_sort(sc, L, T, nv, 64, big);                 /* k >= n: all visible */
    uint16_t* q = malloc(2 * T * H * 576); uint16_t* kv = malloc(2 * L * 576);
    for (int i = 0; i < T * H * 576; ++i) q[i] = bf16();
    for (int i = 0; i < L * 576; ++i) kv[i] = bf16();
    double* out = malloc(sizeof(double) * T * H * 512); double* lse = malloc(sizeof(double) * T * H);
    i1[3] = -1; i1[k + 1] = -1;                                   /* padding inside lists */
    bad |= ora_sparse_mla(q, kv, i1, L, H, k, 0.04, rows, T, out, lse);
    for (int j = 0; j < k; ++j) i1[j] = -1;                       /* a row with no entry */
    bad |= ora_sparse_mla(q, kv, i1, L, H, k, 0.04, rows, 1, out, lse);
    bad |= ora_dense_mla(q, kv, L, H, q_pos0, 0.04, rows, T, out, lse);
    float* x = malloc(sizeof(float) * 5 * 128); uint8_t* c8 = malloc(5 * 128); float* s5 = malloc(sizeof(float) * 5);
    for (int i = 0; i < 5 * 128; ++i) x[i] = (float)((int)(rnd() % 2001) - 1000) * (i < 128 ? 0.f : 0.37f);
    bad |= ora_quantize_e4m3(x, 0, 5, c8, s5);
    int64_t st[4] = {0, 5, 6, 20};
    uint16_t* knew = malloc(2 * 3 * 128); uint16_t* kvnew = malloc(2 * 3 * 576);
    for (int i = 0; i < 3 * 128; ++i) knew[i] = bf16();
    for (int i = 0; i < 3 * 576; ++i) kvnew[i] = bf16();
    uint8_t* k8c = calloc(20 * 128, 1); float* ksc = calloc(20, sizeof(float)); uint16_t* kvc = calloc(20 * 576, 2);
    bad |= ora_decode_append(3, st, knew, 1, kvnew, k8c, ksc, kvc);
    int32_t* win = malloc(4 * T * 5); int32_t* uni = malloc(4 * T * (5 + k));
    bad |= ora_window_indices(T, q_pos0, 5, win);
    bad |= ora_topk_sort(sc, L, T, nv, k, i2);
    bad |= ora_local_selected(i2, T, k, q_pos0, 5, uni);
    /* warm-up on a small real-valued problem, every optional output requested */
    const int n = 6, Lw = 9, HI = 2, Hw = 3;
    double *QI = malloc(8 * n * HI * 128), *ww = malloc(8 * n * HI), *qq = malloc(8 * n * Hw * 576);
    double *KI = malloc(8 * Lw * 128), *kvw = malloc(8 * Lw * 576);
    for (int i = 0; i < n * HI * 128; ++i) QI[i] = ((int)(rnd() % 17) - 8) * 0.125;
    for (int i = 0; i < n * HI; ++i) ww[i] = ((int)(rnd() % 5) - 2) * 0.5;
    for (int i = 0; i < n * Hw * 576; ++i) qq[i] = ((int)(rnd() % 9) - 4) * 0.05;
    for (int i = 0; i < Lw * 128; ++i) KI[i] = ((int)(rnd() % 17) - 8) * 0.125;
    for (int i = 0; i < Lw * 576; ++i) kvw[i] = ((int)(rnd() % 9) - 4) * 0.05;
    int64_t pos[6] = {0, 3, 4, 6, 8, 8};
    double *kl = malloc(8 * n), *lt = malloc(8 * n * Hw), *li = malloc(8 * n), *dq = malloc(8 * n * HI * 128);
    double *dw = malloc(8 * n * HI), *P = malloc(8 * n * Lw), *G = malloc(8 * n * Lw), *dk = malloc(8 * Lw * 128);
    double *klb = malloc(8 * n), *dwb = malloc(8 * n * HI), *dqb = malloc(8 * n * HI * 128), *dqa = malloc(8 * n * HI * 128);
    double *dkb = malloc(8 * Lw * 128), *dka = malloc(8 * Lw * 128);
    bad |= ora_warmup(QI, ww, qq, pos, n, KI, kvw, Lw, HI, Hw, 0.125, 0.04, kl, lt, li, dq, dw, P,
                      G, dk, klb, dwb, dqb, dqa, dkb, dka);
    /* invalid inputs are refused, not run */
    if (ora_topk_sort(sc, L, T, nv, 0, i1) == 0) bad = 1;
    if (ora_window_indices(T, q_pos0, 0, win) == 0) bad = 1;
    free(q8); free(k8); free(qs); free(w); free(ks); free(sc); free(bd); free(i1); free(i2); free(big);
    free(q); free(kv); free(out); free(lse); free(x); free(c8); free(s5); free(knew); free(kvnew);
    free(k8c); free(ksc); free(kvc); free(win); free(uni); free(QI); free(ww); free(qq); free(KI);
    free(kvw); free(kl); free(lt); free(li); free(dq); free(dw); free(P); free(G); free(dk);
    free(klb); free(dwb); free(dqb); free(dqa); free(dkb); free(dka);
    printf(bad ? "oracle driver: failure\n" : "oracle driver ok\n");
    return bad;
}
"""

API_DRIVER = r"""
#include <stdio.h>
#include "dsa.h"

int main(void)
{
    int bad = 0;
    void* p = (void*)(1 << 20);
    float sc[4] = {1, 2, 3, 4};
    int idx[4];
    bad |= dsa_topk(sc, 4, -1, 4, 0, 2, idx, NULL, 0, NULL) != DSA_ERR_INVALID_ARGUMENT;
    bad |= dsa_index_scores(NULL, NULL, NULL, NULL, NULL, 1, 1, 64, 0, 1.f, sc, 1, 0, NULL) != DSA_ERR_INVALID_ARGUMENT;
    bad |= dsa_sparse_mla(p, p, p, 4, 8, 129, 4, 0.1f, p, p, NULL) != DSA_ERR_UNSUPPORTED;
    bad |= dsa_prefill(p, p, p, p, p, p, p, 4, 8, 64, 128, 4, 0, 0.1f, 0.1f, p, p, p, NULL, 0, NULL) != DSA_ERR_WORKSPACE_TOO_SMALL;
    bad |= dsa_decode(4, p, 100, 401, p, p, p, p, p, p, p, 64, 128, 64, 0.1f, 0.1f, p, p, NULL, p, 1 << 20, NULL) != DSA_ERR_INVALID_ARGUMENT;
    bad |= dsa_decode_noalloc(256, p, 131072, 256 * 100000, p, p, p, p, p, p, p, 64, 128, 2048, 0.1f, 0.1f, p, p, NULL, NULL) != DSA_ERR_WORKSPACE_TOO_SMALL;
    int64_t cq[3] = {0, 5, 9}, ck[3] = {0, 4, 9};              /* T_0 > L_0: refused */
    bad |= dsa_prefill_varlen(2, cq, ck, p, p, p, p, p, p, p, 64, 128, 16, 0.1f, 0.1f, p, p, NULL, p, 1 << 30, NULL) != DSA_ERR_INVALID_ARGUMENT;
    bad |= dsa_prefill_varlen_workspace_bytes(2, cq, ck, 64, 128, 16) != 0;
    bad |= dsa_quantize_fp8(p, 3, 4, p, p, NULL) != DSA_ERR_INVALID_ARGUMENT;
    bad |= dsa_indexer_warmup(p, p, p, p, p, p, p, 4, 8, 48, 16, 0, 0.1f, 0.1f, p, p, p, p, NULL, NULL, p, 1 << 20, NULL) != DSA_ERR_UNSUPPORTED;
    bad |= dsa_window_indices(1, 1, 0, 0, idx, NULL) != DSA_ERR_INVALID_ARGUMENT;
    bad |= dsa_local_selected_indices(idx, 1, 1, 0, 1, 1 << 30, idx, NULL) != DSA_ERR_UNSUPPORTED;
    bad |= dsa_prefill_workspace_bytes(131072, 131072, 64, 128, 2048) <= ((size_t)1 << 31);
    bad |= dsa_decode_workspace_bytes(64, 131072, 4199844, 64, 128, 2048) == 0;
    bad |= dsa_indexer_warmup_workspace_bytes(32768, 32768, 64, 128) == 0;
    bad |= dsa_prefill_chunk_rows(131072, 131072) != 4096;
    printf(bad ? "api driver: failure\n" : "api driver ok\n");
    return bad;
}
"""

SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _check_run(exe, tag, cwd):
    r = subprocess.run([exe], capture_output=True, text=True, env=SAN_ENV, cwd=cwd, timeout=300)
    text = r.stdout + r.stderr
    assert r.returncode == 0, text[-3000:]
    assert "AddressSanitizer" not in text and "runtime error" not in text, text[-3000:]
    assert tag in r.stdout


def test_oracle_under_asan_and_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if not gcc:
        pytest.skip("gcc not available")
    src = tmp_path / "driver.c"
    src.write_text(ORACLE_DRIVER)
    exe = tmp_path / "oracle_san"
    cmd = [gcc, "-std=c11", "-O1", "-g", "-fopenmp", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-I", os.path.join(ROOT, "oracle"), str(src), os.path.join(ROOT, "oracle", "oracle.c"),
           "-o", str(exe), "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    _check_run(str(exe), "oracle driver ok", tmp_path)


def test_c_abi_validation_under_asan_and_ubsan(tmp_path):
    from sparse_attention_05_amd import build as hip_build
    if not os.path.exists(hip_build.HIPCC):
        pytest.skip("hipcc not available")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
           "-fno-omit-frame-pointer"]
    objs = []
    for s in hip_build.SOURCES:
        o = tmp_path / (os.path.splitext(s)[0] + ".o")
        cmd = [hip_build.HIPCC, *hip_build.FLAGS, *hip_build.EXTRA.get(s, []), *san, "-g", "-x",
               "hip", "-c", os.path.join(hip_build.CSRC, s), "-o", str(o)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        objs.append(str(o))
    drv = tmp_path / "api_driver.c"
    drv.write_text(API_DRIVER)
    exe = tmp_path / "api_san"
    cmd = [hip_build.HIPCC, "--offload-arch=" + hip_build.ARCH, *san, "-x", "c", str(drv), "-x",
           "none", *objs, "-I", hip_build.INCLUDE, "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    _check_run(str(exe), "api driver ok", tmp_path)
