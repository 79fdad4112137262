"""C-ABI library checks that need no GPU: it loads, exports every symbol the
header declares, sizes its workspaces, and rejects invalid arguments on the host
before anything is enqueued.

The argument-check cases pass placeholder (never dereferenced) pointers; they
only run where no GPU is visible, so a check that wrongly passed could not
reach a device.
"""
import ctypes
import os
import re

import pytest

import draft_head_step_amd as D

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dspark.h")

no_gpu = pytest.mark.skipif(os.path.exists("/dev/kfd"),
                            reason="placeholder-pointer checks run only where no GPU is visible")

OK, EINVAL, EWORKSPACE, EUNSUPPORTED = 0, 1, 2, 3
P = 0x10000          # 16-byte aligned placeholder address, never dereferenced
GREEDY, SAMPLE = 0, 1


def _header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dspark_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = D.lib()
    names = _header_functions()
    assert {"dspark_markov_draft", "dspark_confidence", "dspark_survival", "dspark_schedule"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"{n} declared in dspark.h but not exported"


def test_status_strings():
    L = D.lib()
    assert L.dspark_status_string(0) == b"ok"
    assert L.dspark_status_string(2) == b"workspace too small"
    assert L.dspark_status_string(99) == b"unknown status"


@no_gpu
@pytest.mark.parametrize("args,want", [
    ((0, 5, 4096, 64, 0, GREEDY, 1.0), EINVAL), ((4, 5, 1, 64, 0, GREEDY, 1.0), EINVAL),
    ((4, 5, 4096, 513, 0, GREEDY, 1.0), EINVAL), ((4, 5, 4096, 64, 7, GREEDY, 1.0), EINVAL),
    ((4, 5, 4096, 64, 0, 3, 1.0), EINVAL), ((4, 5, 4096, 64, 0, SAMPLE, 0.0), EINVAL),
])
def test_draft_step_launches_rejects(args, want):
    L = D.lib()
    n = ctypes.c_int(-1)
    assert L.dspark_draft_step_launches(*args, ctypes.byref(n)) == want
    assert L.dspark_draft_step_launches(4, 5, 4096, 64, 0, GREEDY, 1.0, None) == EINVAL
    assert n.value == -1


def test_workspace_queries():
    assert D.dspark_markov_draft_workspace(0, 5, 100, 64) == 0
    assert D.dspark_markov_draft_workspace(4, 5, 1, 64) == 0
    ws = D.dspark_markov_draft_workspace(256, 5, 129280, 512)
    assert ws >= 256 * 8 and ws % 8 == 0
    assert D.dspark_schedule_workspace(0, 7) == 0
    assert D.dspark_schedule_workspace(1 << 20, 16) == 0       # above the candidate limit
    assert D.dspark_schedule_workspace(256, 5) >= 1
    big = D.dspark_schedule_workspace(8192, 7)
    assert big >= 4 * 8192 * 7 * 4 + 256 * (8192 * 7 // 1024) * 4   # keys, ids x2 + digit counts


def _draft(W1=P, W2=P, base=P, anchors=P, R=4, g=5, V=4096, r=64, layout=0, mode=GREEDY, T=1.0,
           u=None, tokens=P, ws=P, ws_bytes=1 << 30, events=None):
    L = D.lib()
    return L.dspark_markov_draft(W1, W2, base, anchors, R, g, V, r, layout, mode, T, u, tokens,
                                 None, ws, ws_bytes, events, None)


@no_gpu
@pytest.mark.parametrize("kw,want", [
    (dict(W1=None), EINVAL), (dict(W2=None), EINVAL), (dict(base=None, mode=SAMPLE, u=P), EINVAL),
    (dict(anchors=None), EINVAL), (dict(tokens=None), EINVAL),
    (dict(R=0), EINVAL), (dict(g=-1), EINVAL), (dict(V=1), EINVAL), (dict(r=0), EINVAL),
    (dict(mode=2), EINVAL), (dict(layout=2), EINVAL), (dict(layout=-1), EINVAL),
    (dict(mode=SAMPLE, u=None), EINVAL),
    (dict(mode=SAMPLE, u=P, T=0.0), EINVAL),
    (dict(mode=SAMPLE, u=P, T=-1.0), EINVAL),
    (dict(mode=SAMPLE, u=P, T=float("inf")), EINVAL),
    (dict(mode=SAMPLE, u=P, T=float("nan")), EINVAL),
    (dict(mode=GREEDY, u=P), EINVAL),
    (dict(W1=P + 4), EINVAL),
    (dict(r=40), EUNSUPPORTED), (dict(r=1024), EUNSUPPORTED),
    # 32-bit byte offsets of one step of one request block
    (dict(g=1, V=1 << 22), EUNSUPPORTED),                       # gamma*V = 2^22, RGV
    (dict(V=(1 << 21) + 32, r=512, layout=1), EUNSUPPORTED),   # ceil(V/32)*32*r > 2^30
    (dict(R=1 << 17, V=4096, layout=1), EUNSUPPORTED),         # ceil(V/32)*R = 2^24, tiled
    (dict(ws=None), EWORKSPACE), (dict(ws_bytes=8), EWORKSPACE), (dict(ws=P + 8), EINVAL),
])
def test_markov_draft_rejects(kw, want):
    assert _draft(**kw) == want
    assert D.lib().dspark_last_error() != b""


@no_gpu
def test_markov_draft_rejects_short_event_list():
    ev = D.StepEvents(None, None, 3)
    assert _draft(events=ctypes.byref(ev)) == EINVAL


@no_gpu
@pytest.mark.parametrize("idx", range(6))
def test_confidence_rejects_null(idx):
    # h, W1, anchors, tokens, w_conf and conf are required (sts_temp and surv are optional)
    args = [P] * 6
    args[idx] = None
    h, W1, anchors, tokens, w_conf, conf = args
    L = D.lib()
    assert L.dspark_confidence(h, W1, anchors, tokens, w_conf, None, 4, 5, 256, 4096, 64, conf,
                               None, None) == EINVAL


@no_gpu
def test_confidence_rejects_sizes():
    L = D.lib()
    assert L.dspark_confidence(P, P, P, P, P, None, 4, 5, 0, 4096, 64, P, None, None) == EINVAL


@no_gpu
def test_survival_rejects():
    L = D.lib()
    assert L.dspark_survival(None, 4, 5, P, None) == EINVAL
    assert L.dspark_survival(P, 0, 5, P + 64, None) == EINVAL
    assert L.dspark_survival(P, 4, 5, P, None) == EINVAL       # aliasing


@no_gpu
def test_w2_store_from_rv_rejects():
    L = D.lib()
    assert L.dspark_w2_store_from_rv(None, 512, 1000, P + (1 << 24), None) == EINVAL
    assert L.dspark_w2_store_from_rv(P, 512, 1000, None, None) == EINVAL
    assert L.dspark_w2_store_from_rv(P, 0, 1000, P + (1 << 24), None) == EINVAL
    assert L.dspark_w2_store_from_rv(P, 512, -1, P + (1 << 24), None) == EINVAL
    # the two arrays overlap (1000 x 512 bf16 = 1,024,000 bytes each)
    assert L.dspark_w2_store_from_rv(P, 512, 1000, P + 1_000_000, None) == EINVAL
    assert L.dspark_w2_store_from_rv(P + 1_000_000, 512, 1000, P, None) == EINVAL
    assert L.dspark_w2_store_from_rv(P, 64 * 65535 + 1, 4, P + (1 << 40), None) == EUNSUPPORTED
    assert L.dspark_w2_store_from_rv(P, 16, 1 << 30, P + (1 << 40), None) == EUNSUPPORTED


@no_gpu
@pytest.mark.parametrize("kw,want", [
    (dict(surv=None), EINVAL), (dict(sps=None), EINVAL), (dict(lengths=None), EINVAL),
    (dict(R=0), EINVAL), (dict(B_max=23), EINVAL),
    (dict(R=1 << 21, g=8, B_max=(1 << 21) * 9), EUNSUPPORTED),
    (dict(ws=None), EWORKSPACE), (dict(ws_bytes=1), EWORKSPACE),
])
def test_schedule_rejects(kw, want):
    a = dict(surv=P, sps=P, R=4, g=5, B_max=24, lengths=P, ws=P, ws_bytes=1 << 20)
    a.update(kw)
    L = D.lib()
    st = L.dspark_schedule(a["surv"], a["sps"], a["R"], a["g"], a["B_max"], a["lengths"], None,
                           None, a["ws"], a["ws_bytes"], None)
    assert st == want


@no_gpu
@pytest.mark.parametrize("kw,want", [
    (dict(mode=3), EINVAL), (dict(mode=-1), EINVAL),
    (dict(mode=2, capacity=-1), EINVAL),
    (dict(mode=1, sps=None), EINVAL), (dict(mode=0, sps=None), EINVAL),
    (dict(mode=1, B_max=23), EINVAL),
    (dict(mode=2, surv=None), EINVAL), (dict(mode=2, lengths=None), EINVAL),
    (dict(mode=2, R=0), EINVAL),
    (dict(mode=2, R=1 << 21, g=8), EUNSUPPORTED),
    (dict(mode=2, ws=None), EWORKSPACE), (dict(mode=1, ws_bytes=1), EWORKSPACE),
])
def test_schedule_ex_rejects(kw, want):
    a = dict(surv=P, sps=P, R=4, g=5, B_max=24, mode=0, capacity=10, lengths=P, ws=P,
             ws_bytes=1 << 20)
    a.update(kw)
    L = D.lib()
    st = L.dspark_schedule_ex(a["surv"], a["sps"], a["R"], a["g"], a["B_max"], a["mode"],
                              a["capacity"], a["lengths"], None, None, a["ws"], a["ws_bytes"],
                              None)
    assert st == want
    assert L.dspark_last_error() != b""


@no_gpu
@pytest.mark.parametrize("idx", range(5))
def test_verify_pack_rejects_null(idx):
    args = [P] * 5   # anchors, tokens, lengths, flat_tokens, cu_seqlens (pos0 / pos / req optional)
    args[idx] = None
    an, tk, ln, ft, cu = args
    assert D.lib().dspark_verify_pack(an, tk, ln, None, 4, 5, ft, None, None, cu, None) == EINVAL


@no_gpu
def test_verify_rejects_sizes_and_nulls():
    L = D.lib()
    assert L.dspark_verify_pack(P, P, P, None, 0, 5, P, None, None, P, None) == EINVAL
    assert L.dspark_verify_pack(P, P, P, None, 1 << 30, 4, P, None, None, P, None) == EUNSUPPORTED
    assert L.dspark_verify_greedy(P, P, P, 4, 5, 0, P, P, P, None) == EINVAL
    for i in range(6):
        a = [P] * 6
        a[i] = None
        assert L.dspark_verify_greedy(a[0], a[1], a[2], 4, 5, 100, a[3], a[4], a[5], None) == EINVAL


@no_gpu
@pytest.mark.parametrize("kw,want", [
    (dict(d=None), EINVAL), (dict(t=None), EINVAL), (dict(o=None), EINVAL),
    (dict(n=0), EINVAL), (dict(V=0), EINVAL),
    (dict(T=0.0), EINVAL), (dict(T=-1.0), EINVAL), (dict(T=float("inf")), EINVAL),
    (dict(T=float("nan")), EINVAL),
])
def test_accept_prob_rejects(kw, want):
    a = dict(d=P, t=P, n=4, V=100, T=1.0, o=P)
    a.update(kw)
    assert D.lib().dspark_accept_prob(a["d"], a["t"], a["n"], a["V"], a["T"], a["o"], None) == want


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setenv("DSPARK_LIB", str(tmp_path / "missing.so"))
    monkeypatch.setattr(D, "_LIB", None)
    with pytest.raises(ImportError):
        D.lib()


def test_tiled_layout_roundtrip():
    import numpy as np
    from draft_head_step_amd.inputs import from_tiled, to_tiled
    x = np.random.default_rng(0).standard_normal((5, 3, 70)).astype(np.float32)
    t = to_tiled(x)
    assert t.shape == (3, 3, 32, 5)
    # element (m, k, v) at ((k * C + v // 32) * 32 + v % 32) * R + m
    flat = t.reshape(-1)
    for (m, k, v) in [(0, 0, 0), (4, 2, 69), (2, 1, 33), (3, 0, 31)]:
        assert flat[((k * 3 + v // 32) * 32 + v % 32) * 5 + m] == x[m, k, v]
    assert np.array_equal(from_tiled(t, 70), x)
    assert np.all(t[:, 2, 6:, :] == 0)


def test_library_matches_the_tree_sources():
    from draft_head_step_amd import build as B
    assert D.lib().dspark_source_hash().decode() == B.source_hash()


def test_stale_library_is_refused(monkeypatch):
    # A library built from other sources (its embedded hash differs from the
    # tree's) must not load.
    monkeypatch.setattr(D, "_LIB", None)
    monkeypatch.setattr(D, "_tree_hash", lambda: "0" * 32)
    with pytest.raises(ImportError, match="other sources"):
        D.lib()
    monkeypatch.setattr(D, "_LIB", None)


def test_source_hash_follows_every_source_file(tmp_path, monkeypatch):
    # Changing any kernel source, internal header or the public header changes the hash.
    from draft_head_step_amd import build as B
    h0 = B.source_hash()
    files = B.source_files()
    assert any(f.endswith("dspark.h") for f in files)
    assert any(f.endswith("markov_step.hip") for f in files)
    real_open = open

    def fake_open(path, mode="r", *a, **k):
        fh = real_open(path, mode, *a, **k)
        if path == files[0] and "b" in mode:
            data = fh.read() + b"// changed"
            fh.close()
            import io
            return io.BytesIO(data)
        return fh
    monkeypatch.setattr("builtins.open", fake_open)
    assert B.source_hash() != h0


@no_gpu
@pytest.mark.parametrize("kw,want", [
    (dict(W1=None), EINVAL), (dict(tokens=None), EINVAL), (dict(R=0), EINVAL),
    (dict(mode=SAMPLE, u=None), EINVAL), (dict(r=40), EUNSUPPORTED),
    (dict(R=4097, g=8), EUNSUPPORTED),          # R * gamma above the static scratch
    (dict(R=32768, g=1, V=64, r=16), None),      # at the limit: passes the size check
])
def test_markov_draft_noalloc_rejects(kw, want):
    a = dict(W1=P, W2=P, base=P, anchors=P, R=4, g=5, V=4096, r=64, layout=0, mode=GREEDY,
             T=1.0, u=None, tokens=P)
    a.update(kw)
    L = D.lib()
    if want is None:
        # only the size arithmetic is exercised: the workspace query fits the array
        need = D.dspark_markov_draft_workspace(a["R"], a["g"], a["V"], a["r"])
        assert need <= 4 << 20
        return
    st = L.dspark_markov_draft_noalloc(a["W1"], a["W2"], a["base"], a["anchors"], a["R"], a["g"],
                                       a["V"], a["r"], a["layout"], a["mode"], a["T"], a["u"],
                                       a["tokens"], None)
    assert st == want
    assert L.dspark_last_error() != b""


def test_scratch_check_recognises_counted_wait_kernels():
    from draft_head_step_amd import build as B
    rem = ("x.hip:1:1: remark: Function Name: _ZN6dspark12_GLOBAL__N_125markov_step_ksplit_kernelILi4ELi1ELi2ELb0EEEvPKt [-Rpass-analysis=kernel-resource-usage]\n"
           "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 16 [-Rpass-analysis=kernel-resource-usage]\n"
           "x.hip:1:1: remark: Function Name: _ZN6dspark12_GLOBAL__N_118markov_step_kernelILi512ELi8ELi0ELi2ELb1ELi1EEEvPKt [-Rpass-analysis=kernel-resource-usage]\n"
           "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 64 [-Rpass-analysis=kernel-resource-usage]\n"
           "x.hip:1:1: remark: Function Name: _ZN6dspark12_GLOBAL__N_118markov_step_kernelILi256ELi8ELi1ELi2ELb0ELi1EEEvPKt [-Rpass-analysis=kernel-resource-usage]\n"
           "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 32 [-Rpass-analysis=kernel-resource-usage]\n"
           "x.hip:1:1: remark: Function Name: _ZN6dspark12_GLOBAL__N_118markov_step_kernelILi512ELi4ELi0ELi2ELb0ELi1EEEvPKt [-Rpass-analysis=kernel-resource-usage]\n"
           "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 8 [-Rpass-analysis=kernel-resource-usage]\n"
           "x.hip:1:1: remark: Function Name: _ZN6dspark12_GLOBAL__N_129markov_step_ksplit_fin_kernelILi4ELi1ELi2EEEvPKt [-Rpass-analysis=kernel-resource-usage]\n"
           "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 4 [-Rpass-analysis=kernel-resource-usage]\n")
    bad = B.scratch_offenders(rem)
    # the K-split (also the fused step's last-step one) and the rank-512 plain
    # kernel without bias output count their waits; the bias-output (Lb1E) and
    # register-staged rank-256 ones do not
    assert len(bad) == 3 and "ksplit" in bad[0] and "ILi512ELi4E" in bad[1]
    assert "ksplit_fin" in bad[2]


def _step(**kw):
    a = dict(W1=P, W2=P, base=P, anchors=P, R=4, g=5, V=4096, r=64, layout=0, mode=GREEDY,
             T=1.0, u=None, h=P, w=P, sts=None, d=256, sps=P, B_max=24, tokens=P, conf=P,
             surv=P, lengths=P, order=None, info=None, ws=0x100000, ws_bytes=1 << 30)
    a.update(kw)
    L = D.lib()
    return L.dspark_draft_step(a["W1"], a["W2"], a["base"], a["anchors"], a["R"], a["g"], a["V"],
                               a["r"], a["layout"], a["mode"], a["T"], a["u"], a["h"], a["w"],
                               a["sts"], a["d"], a["sps"], a["B_max"], a["tokens"], a["conf"],
                               a["surv"], a["lengths"], a["order"], a["info"], a["ws"],
                               a["ws_bytes"], None, None)


@no_gpu
@pytest.mark.parametrize("kw,want", [
    (dict(W1=None), EINVAL), (dict(h=None), EINVAL), (dict(w=None), EINVAL),
    (dict(sps=None), EINVAL), (dict(conf=None), EINVAL), (dict(surv=None), EINVAL),
    (dict(lengths=None), EINVAL), (dict(d=0), EINVAL), (dict(B_max=23), EINVAL),
    (dict(mode=SAMPLE, u=None), EINVAL), (dict(r=40), EUNSUPPORTED),
    (dict(d=30), EUNSUPPORTED), (dict(w=P + 4), EUNSUPPORTED),
    (dict(R=1 << 21, g=8, B_max=9 << 21), EUNSUPPORTED),
    (dict(ws=None), EWORKSPACE), (dict(ws_bytes=16), EWORKSPACE), (dict(ws=0x100000 + 16), EINVAL),
])
def test_draft_step_rejects(kw, want):
    assert _step(**kw) == want
    assert D.lib().dspark_last_error() != b""


@no_gpu
def test_schedule_rejects_tau_overflow_sizes():
    # R * (1 + gamma) must stay below 2^24 (gamma = 1, R = 2^23 has 2^23 candidates
    # but a fixed-point tau that could reach 2^64).
    L = D.lib()
    R = 1 << 23
    assert L.dspark_schedule(P, P, R, 1, 2 * R, P, None, None, P, 1 << 30, None) == EUNSUPPORTED
    assert D.dspark_schedule_workspace(R, 1) == 0
    assert D.dspark_schedule_workspace(R - 1, 1) > 0


def _rnn(**kw):
    a = dict(W1=P, W2=P, U=P, b=P, base=P, h=P, anchors=P, R=4, g=5, V=4096, r=64, d=256,
             layout=0, mode=GREEDY, T=1.0, u=None, tokens=P, state=None, ws=0x100000,
             ws_bytes=1 << 30)
    a.update(kw)
    return D.lib().dspark_rnn_draft(a["W1"], a["W2"], a["U"], a["b"], a["base"], a["h"],
                                    a["anchors"], a["R"], a["g"], a["V"], a["r"], a["d"],
                                    a["layout"], a["mode"], a["T"], a["u"], a["tokens"],
                                    a["state"], a["ws"], a["ws_bytes"], None, None)


@no_gpu
@pytest.mark.parametrize("kw,want", [
    (dict(U=None), EINVAL), (dict(b=None), EINVAL), (dict(h=None), EINVAL), (dict(d=0), EINVAL),
    (dict(d=30), EUNSUPPORTED), (dict(U=P + 4), EUNSUPPORTED), (dict(h=P + 8), EUNSUPPORTED),
    (dict(R=1 << 20, g=16, r=128), EUNSUPPORTED),
    (dict(r=512, d=(1 << 22) - 1016), EUNSUPPORTED),
    (dict(ws=None), EWORKSPACE), (dict(ws_bytes=16), EWORKSPACE), (dict(ws=0x100000 + 16), EINVAL),
])
def test_rnn_draft_rejects(kw, want):
    assert _rnn(**kw) == want
    assert D.lib().dspark_last_error() != b""


@no_gpu
def test_rnn_workspace_holds_the_pre_activation_partials():
    # At the DeepSeek-V4 shape the pre-activations are split over K into 3
    # partial sums of R * gamma * 2r floats (80 tiles, about one workgroup per
    # CU); a small shape keeps one.
    big = D.dspark_rnn_draft_workspace(256, 5, 129280, 512, 7168)
    assert big >= 3 * 256 * 5 * 1024 * 4
    small = D.dspark_rnn_draft_workspace(4, 5, 4096, 64, 256)
    assert 4 * 5 * 128 * 4 <= small < 2 * 4 * 5 * 128 * 4 + (1 << 20)
