"""Host logic of bench.py (no GPU): the one-GPU guard, the byte and flop counts
behind the reported rooflines, and the validity check of the committed counter
summaries."""
import dataclasses
import os
import re
import subprocess
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from long_context_decode_predict_amd import workloads  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def test_admitted_bytes_counts_the_partial_last_block():
    # two rows: 130 tokens (blocks 0, 1 full, block 2 holds 2 tokens) and 128 (two full)
    w = workloads.custom("ab", B=2, H=2, d=64, T=130, kv_dtype=torch.bfloat16)
    cnt = np.array([[2, 1], [2, 0]])
    idx = np.zeros((2, 2, 4), dtype=np.int64)
    idx[0, 0, :2] = [0, 2]  # ends on the partial block: 64 + 2 tokens
    idx[0, 1, :1] = [1]     # 64 tokens
    idx[1, 0, :2] = [0, 1]  # 128 tokens (row of 128: no partial block)
    got = bench.admitted_bytes(w, cnt, idx, [130, 128])
    assert got == 2 * (66 + 64 + 128) * 64 * 2  # K and V, bf16


def test_prefill_flops_closed_form():
    w = workloads.PREFILL_WORKLOADS["prefill_b4_h16_d128_t8k_bf16"]
    T = w.T_q
    assert w.T_k == T
    assert bench.prefill_flops(w) == 4 * w.d * (T * (T + 1) // 2) * w.B * w.H
    # a chunk of 100 queries after a prefix of 900 keys: 100 * 900 + 100 * 101 / 2 pairs
    c = dataclasses.replace(w, T_q=100, T_k=1000)
    assert bench.prefill_flops(c) == 4 * w.d * (100 * 900 + 5050) * w.B * w.H


def test_source_hash_ignores_comments_and_layout(tmp_path, monkeypatch):
    csrc = tmp_path / "long_context_decode_predict_amd" / "csrc"
    csrc.mkdir(parents=True)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (csrc / "a.hip").write_text("int f(int x) {\n    return x + 1;  // one\n}\n")
    h0 = bench.attn_source_sha(("a.hip",))
    (csrc / "a.hip").write_text("/* header */\nint f(int x) { return x + 1; }   // other\n")
    assert bench.attn_source_sha(("a.hip",)) == h0
    (csrc / "a.hip").write_text("int f(int x) { return x + 2; }\n")
    assert bench.attn_source_sha(("a.hip",)) != h0


def test_committed_counter_summaries_parse(monkeypatch):
    """Every attention / prefill profile summary names its workload and carries the
    traffic and source hash that bench.py reads; a different hash makes the traffic
    null instead of stale."""
    names = sorted(os.listdir(os.path.join(ROOT, "profiles")))
    attn = [n for n in names if n.startswith("attn_partial_")]
    pre = [n for n in names if n.startswith("prefill_attn_")]
    assert attn and pre
    for n in attn + pre:
        wl = n.split("_", 2)[2][:-3]
        assert wl in workloads.WORKLOADS or wl in workloads.PREFILL_WORKLOADS, n
        text = open(os.path.join(ROOT, "profiles", n)).read()
        assert "rocprofv3" in text and "traffic_bytes_per_launch:" in text
        sha = [ln.split(":", 1)[1].strip() for ln in text.splitlines()
               if ln.startswith("attn_source_sha256:")]
        assert len(sha) == 1 and len(sha[0]) == 64
    wl = attn[0][len("attn_partial_"):-3]
    monkeypatch.setattr(bench, "attn_source_sha", lambda sources=None: "0" * 64)
    assert bench.counter_traffic(wl) is None


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_metadata_bytes_per_block(name):
    w = workloads.WORKLOADS[name]
    lens = workloads.row_lengths(w)
    blocks = w.kv_heads * sum((t + 63) // 64 for t in lens)
    assert bench.meta_bytes(w, lens) == blocks * (w.d + 2) * 4


def test_step_stats_median_and_spread():
    st = bench.step_stats([4.0, 1.0, 3.0, 2.0, 100.0], total_ms=110.0)
    assert st["median"] == 3.0 and st["min"] == 1.0 and st["max"] == 100.0
    assert st["mean"] == 22.0 and st["n"] == 5
    assert st["p10"] <= st["median"] <= st["p90"]


def test_cpu_baseline_threads_and_host_counts():
    cpus = bench.host_cpus()
    assert cpus["os_cpu_count"] == os.cpu_count()
    n = bench.host_threads()
    assert 1 <= n <= bench.CPU_SHARE
    assert n <= (cpus["affinity"] or os.cpu_count())


def test_read_probe_library_exports_and_rejects_bad_sizes():
    """libeta_probe.so is built beside libeta.so and refuses invalid arguments before
    any launch (a size that is not whole chunks, null or misaligned pointers)."""
    import ctypes

    from long_context_decode_predict_amd.build import PROBE_LIB_PATH, ensure_built
    ensure_built()
    L = ctypes.CDLL(PROBE_LIB_PATH)
    text = open(os.path.join(os.path.dirname(PROBE_LIB_PATH), "..", "include", "eta_probe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    declared = sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(eta_probe_\w+)\s*\(", text, flags=re.M)))
    assert declared == ["eta_probe_pair_read", "eta_probe_stream_read"], declared
    for n in declared:
        assert hasattr(L, n), n
    f = L.eta_probe_stream_read
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                  ctypes.c_void_p]
    fake = 0x100000
    assert f(fake, 32768 + 16, 1, fake, None) == -1
    assert f(fake, 0, 1, fake, None) == -1
    assert f(None, 32768, 1, fake, None) == -1
    assert f(fake, 32768, 0, None, None) == -1
    assert f(fake + 8, 32768, 1, fake, None) == -1
    g = L.eta_probe_pair_read
    g.restype = ctypes.c_int
    g.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                  ctypes.c_void_p]
    assert g(fake, fake, 16384 + 16, fake, None) == -1
    assert g(fake, fake, 0, fake, None) == -1
    assert g(None, fake, 16384, fake, None) == -1
    assert g(fake, None, 16384, fake, None) == -1
    assert g(fake, fake, 16384, None, None) == -1
    assert g(fake, fake + 8, 16384, fake, None) == -1


def test_interleaved_cache_views_hold_the_same_rows():
    """bench.interleave_kv moves a dense cache into one buffer with K and V interleaved
    block by block: the block views it hands the library have the block stride the C
    ABI expects (128*d), and every unit's rows read back through them equal the
    separate buffers' rows (host tensors; no library call)."""
    from long_context_decode_predict_amd import _lib
    B, Hk, Tc, d = 2, 3, 192, 16
    K = torch.randn(B, Hk, Tc, d)
    V = torch.randn(B, Hk, Tc, d)
    data = {"K": K.clone(), "V": V.clone()}
    bench.interleave_kv(data)
    Kb, Vb = bench.kv_of(data)
    assert data["K"] is None and data["V"] is None
    assert _lib.kv_block_view(Kb) and _lib.kv_block_stride(Kb) == 2 * 64 * d
    assert Vb.data_ptr() - Kb.data_ptr() == 64 * d * K.element_size()
    assert _lib.kv_dims(Kb) == (B, Hk, Tc, d, 0)
    for b in range(B):
        for k in range(Hk):
            Ku, Vu = bench.unit_kv(data, b, k, 150)
            assert torch.equal(Ku, K[b, k, :150]) and torch.equal(Vu, V[b, k, :150])
