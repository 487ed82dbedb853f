"""Host-only checks of the C ABI: the library loads, exports every symbol the
header declares, sizes its buffers by the closed forms, and rejects bad
arguments before enqueueing anything.  No kernel is launched here."""
import ctypes

import pytest

import oracle as orc

BIG = 1 << 40


def test_exports_every_declared_symbol(lh):
    names = lh.declared_symbols()
    assert set(names) >= {"lh_query", "lh_forward", "lh_backward", "lh_attention_forward", "lh_saved_layout",
                          "lh_status_string", "lh_last_error", "lh_attention_backward", "lh_layer_query",
                          "lh_layer_saved_layout", "lh_layer_forward", "lh_layer_backward", "lh_stage_name",
                          "lh_timing_begin", "lh_timing_end"}
    lib = lh.library()
    for n in names:
        assert hasattr(lib, n), n
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


@pytest.mark.parametrize("B,H,N,d,L,p,k,io", [
    (1, 2, 1024, 64, 3, 4, 64, "f32"), (1, 8, 98304, 128, 3, 4, 768, "bf16"), (1, 8, 524288, 128, 3, 4, 4096, "bf16"),
    (1, 8, 1048576, 128, 4, 4, 4096, "bf16"), (1, 8, 8192, 128, 3, 4, 64, "bf16"), (1, 2, 1024, 64, 3, 4, 1024, "f32"),
    (2, 3, 96, 64, 1, 4, 5, "f32"), (1, 1, 1000000, 128, 4, 4, 4096, "bf16"), (1, 1, 64, 128, 4, 2, 0, "bf16")])
def test_query_matches_closed_form(lh, B, H, N, d, L, p, k, io):
    st, S, saved, fws, bws = lh.lh_query(B, H, N, d, L, p, k, io)
    assert st == 0, lh.lh_last_error()
    sizes = orc.level_sizes(N, L, p)
    assert S == sizes[-1] + orc.budget(N, L, p, k)
    st, lay = lh.lh_saved_layout(B, H, N, d, L, p, k, io)
    assert st == 0
    assert lay["S"] == S and lay["P"] == sum(sizes) and lay["E"] == sum(sizes[:-1])
    assert lay["Sv"] == (S + 63) // 64 * 64
    es = 2 if io == "bf16" else 4
    BH = B * H
    order = ["scores", "flags", "slot", "coords", "qt", "kt", "vt", "ot", "lse"]
    need = {"scores": 8 * BH * lay["P"], "flags": BH * lay["P"], "slot": 4 * BH * lay["P"], "coords": 4 * BH * S,
            "qt": es * BH * lay["Sv"] * d, "kt": es * BH * lay["Sv"] * d, "vt": es * BH * lay["Sv"] * d,
            "ot": 4 * BH * S * d, "lse": 4 * BH * S}
    for a, b in zip(order, order[1:] + ["total"]):
        assert lay[a] % 256 == 0
        assert lay[b] - lay[a] >= need[a]           # arrays do not overlap
    assert saved == lay["total"]
    # backward workspace: dQ~, dK~, dV~ in fp32, plus dO~ (fp32 in fp32 mode; bf16 rows padded to Sv and the
    # (LSE log2 e, delta) row pairs in bf16 mode)
    need_bws = 3 * 4 * BH * S * d + (4 * BH * S * d if io == "f32" else 2 * BH * lay["Sv"] * d + 8 * BH * lay["Sv"])
    assert fws > 0 and bws >= need_bws


def test_page_example_S_through_abi(lh):
    st, S, *_ = lh.lh_query(1, 1, 10 ** 6, 128, 4, 4, 4096, "bf16")
    assert st == 0 and S == 64777


@pytest.mark.parametrize("args,status", [
    ((1, 1, 1000, 64, 3, 4, 8, "f32"), 2),       # 16 does not divide 1000
    ((1, 1, 1024, 96, 3, 4, 8, "f32"), 3),       # d unsupported
    ((1, 1, 1024, 64, 0, 4, 8, "f32"), 1),       # L < 1
    ((1, 1, 1024, 64, 3, 1, 8, "f32"), 1),       # p < 2
    ((1, 1, 1024, 64, 3, 4, -1, "f32"), 1),      # k < 0
    ((0, 1, 1024, 64, 3, 4, 8, "f32"), 1),       # B < 1
    ((1, 1, 0, 64, 3, 4, 8, "f32"), 1),          # N < 1
    ((1, 1, 16, 64, 4, 4, 8, "f32"), 2),         # p^(L-1) > N
    ((1, 1, 1 << 25, 128, 3, 4, 8, "f32"), 3),   # N*d >= 2^31
])
def test_query_rejects(lh, args, status):
    st, *_ = lh.lh_query(*args)
    assert st == status
    assert lh.lh_last_error()
    assert lh.lh_status_string(st) != "unknown status"


def test_huge_topk_selects_everything(lh):
    st, S, *_ = lh.lh_query(1, 1, 1024, 64, 3, 4, BIG, "f32")
    assert st == 0 and S == 1344


@pytest.mark.parametrize("topk", [BIG - 1, (1 << 62), (1 << 63) - 1, 1 << 24, (1 << 24) - 1])
def test_budget_saturates_without_overflow(lh, topk):
    """(L-1) p k beyond every int64 for a large p: the budget is capped at the
    candidates without forming the product, so S = |P| (no wrap-around).  At
    p = 2^24, L = 2, N = 2^24 there are E = 2^24 candidates and one coarsest
    entry; k = 1 already reaches the cap."""
    N, p = 1 << 24, 1 << 24
    st, S, saved, fws, bws = lh.lh_query(1, 1, N, 64, 2, p, topk, "bf16")
    assert st == 0, lh.lh_last_error()
    assert S == N + 1
    assert 0 < saved < (1 << 40) and 0 < fws < (1 << 40) and 0 < bws < (1 << 40)


def test_budget_below_the_cap(lh):
    """Below the cap the budget is exactly (L-1) p k, also for a large p."""
    N, L, p = 1 << 20, 2, 1 << 10   # E = 2^20 candidates, 2^10 coarsest entries
    for k in (0, 1, 1023):
        st, S, *_ = lh.lh_query(1, 1, N, 64, L, p, k, "bf16")
        assert st == 0 and S == (N >> 10) + (L - 1) * p * k
    st, S, *_ = lh.lh_query(1, 1, N, 64, L, p, 1024, "bf16")
    assert st == 0 and S == (N >> 10) + N


def test_forward_validation_before_launch(lh):
    """Every one of these fails validation on the host; nothing is enqueued."""
    B, H, N, d, L, p, k = 1, 2, 1024, 64, 3, 4, 64
    st, S, saved, fws, bws = lh.lh_query(B, H, N, d, L, p, k, "f32")
    fake = 1 << 20                     # aligned, never dereferenced
    # null pointer
    assert lh.lh_forward(None, fake, fake, fake, "f32", B, H, N, d, L, p, k, "f32", fake, saved, fake, fws) == 1
    # misaligned pointer
    assert lh.lh_forward(fake + 4, fake, fake, fake, "f32", B, H, N, d, L, p, k, "f32", fake, saved, fake, fws) == 1
    # saved buffer too small
    assert lh.lh_forward(fake, fake, fake, fake, "f32", B, H, N, d, L, p, k, "f32", fake, saved - 1, fake, fws) == 4
    assert "saved" in lh.lh_last_error()
    # workspace too small
    assert lh.lh_forward(fake, fake, fake, fake, "f32", B, H, N, d, L, p, k, "f32", fake, saved, fake, fws - 1) == 4
    # bad output dtype (raw call: the binding itself refuses unknown dtypes)
    assert lh.library().lh_forward(fake, fake, fake, fake, 7, B, H, N, d, L, p, k, 0, fake, saved, fake, fws,
                                   None) == 1
    # divisibility is checked before anything else
    assert lh.lh_forward(fake, fake, fake, fake, "f32", B, H, 1000, d, L, p, k, "f32", fake, saved, fake, fws) == 2
    # backward: workspace too small, null gradient
    assert lh.lh_backward(fake, fake, fake, fake, "f32", fake, saved, fake, fake, fake, "f32", B, H, N, d, L, p, k,
                          "f32", fake, bws - 1) == 4
    assert lh.lh_backward(fake, fake, fake, fake, "f32", fake, saved, None, fake, fake, "f32", B, H, N, d, L, p, k,
                          "f32", fake, bws) == 1
    # dense attention: unsupported d
    assert lh.lh_attention_forward(fake, fake, fake, fake, None, 1, 128, 80, "bf16") == 3
    # dense attention backward: bf16 needs S % 64 == 0, workspace size, null lse, misaligned gradient
    bw = lh.attention_backward_ws_bytes(2, 128, "bf16")
    assert bw == 8 * 2 * 128 and lh.attention_backward_ws_bytes(2, 100, "f32") == 4 * 2 * 100
    args = (fake, fake, fake, fake, fake, fake, fake, fake, fake)
    assert lh.lh_attention_backward(*args, 2, 100, 64, "bf16", fake, 8 * 2 * 100) == 3
    assert lh.lh_attention_backward(*args, 2, 128, 64, "bf16", fake, bw - 1) == 4
    assert lh.lh_attention_backward(fake, fake, fake, fake, None, fake, fake, fake, fake, 2, 128, 64, "bf16", fake,
                                    bw) == 1
    assert lh.lh_attention_backward(fake, fake, fake, fake, fake, fake, fake + 8, fake, fake, 2, 100, 64, "f32",
                                    fake, 800) == 1
    assert lh.lh_attention_backward(*args, 2, 128, 96, "bf16", fake, bw) == 3


def test_stage_timing_host_side(lh):
    """Stage names and enum size match the header; timing with no calls in
    between records nothing; bad output arrays are rejected.  (No GPU work.)"""
    import re
    hdr = open(lh.HEADER).read()
    names = [lh.lh_stage_name(i) for i in range(lh.STAGE_COUNT)]
    assert names == ["pool_score", "topk", "gather", "attn_fwd", "scatter", "scatter_bwd", "attn_bwd_dq",
                     "attn_bwd_dkdv", "pool_bwd", "proj", "out_proj", "out_proj_bwd", "proj_bwd"]
    assert lh.lh_stage_name(lh.STAGE_COUNT) == "unknown"
    assert int(re.search(r"LH_STAGE_COUNT\s*=\s*(\d+)", hdr).group(1)) == lh.STAGE_COUNT
    assert lh.lh_timing_begin() == 0
    st, stages = lh.lh_timing_end()
    assert st == 0 and all(ms == 0.0 and s == 0 for ms, s in stages.values())
    assert lh.library().lh_timing_end(None, None, 3) == 1
    assert lh.library().lh_timing_end(None, None, 0) == 0


@pytest.mark.parametrize("B,H,N,dm,d,io", [(1, 8, 524288, 1024, 128, "bf16"), (2, 3, 1040, 192, 64, "f32"),
                                           (1, 2, 1024, 128, 64, "f32"), (2, 3, 1040, 192, 64, "bf16")])
def test_layer_query_and_layout(lh, B, H, N, dm, d, io):
    """The layer's saved buffer holds Q, K, V, O in the head layout and then the
    attention's own saved buffer; the workspaces cover the attention's."""
    L, p, k = 3, 4, 32
    st, S, saved, fws, bws = lh.lh_layer_query(B, H, N, dm, d, L, p, k, io)
    assert st == 0, lh.lh_last_error()
    st2, S2, isaved, ifws, ibws = lh.lh_query(B, H, N, d, L, p, k, io)
    assert st2 == 0 and S == S2
    st, lay = lh.lh_layer_saved_layout(B, H, N, dm, d, L, p, k, io)
    assert st == 0
    head = (2 if io == "bf16" else 4) * B * H * N * d
    order = ["q", "k", "v", "o", "inner"]
    for a, b in zip(order, order[1:]):
        assert lay[a] % 256 == 0 and lay[b] - lay[a] >= head
    assert lay["inner_bytes"] == isaved and lay["inner"] + isaved <= lay["total"] == saved
    assert fws == ifws
    assert bws >= 4 * head + ibws


def test_layer_validation_before_launch(lh):
    """Bad layer arguments fail on the host; nothing is enqueued."""
    B, H, N, dm, d, L, p, k = 1, 2, 1024, 128, 64, 3, 4, 64
    st, S, saved, fws, bws = lh.lh_layer_query(B, H, N, dm, d, L, p, k, "f32")
    assert st == 0
    fake = 1 << 20
    assert lh.lh_layer_query(B, H, N, 96, d, L, p, k, "f32")[0] == 3        # d_model not a multiple of 64
    assert lh.lh_layer_query(B, H, N, dm, 96, L, p, k, "f32")[0] == 3       # d unsupported
    assert lh.lh_layer_query(B, H, 1000, dm, d, L, p, k, "f32")[0] == 2     # p^(L-1) does not divide N
    ws6 = (fake,) * 6
    assert lh.lh_layer_forward(*ws6, "f32", B, H, N, dm, d, L, p, k, "f32", fake, saved - 1, fake, fws) == 4
    assert lh.lh_layer_forward(*ws6, "f32", B, H, N, dm, d, L, p, k, "f32", fake, saved, fake, fws - 1) == 4
    assert lh.lh_layer_forward(None, *ws6[1:], "f32", B, H, N, dm, d, L, p, k, "f32", fake, saved, fake, fws) == 1
    assert lh.lh_layer_forward(*ws6[:5], fake + 8, "f32", B, H, N, dm, d, L, p, k, "f32", fake, saved, fake,
                               fws) == 1
    assert lh.library().lh_layer_forward(*ws6, 7, B, H, N, dm, d, L, p, k, 0, fake, saved, fake, fws, None) == 1
    # backward: every call below fails validation (workspace, saved size, null or misaligned gradient, dtype)
    head = (fake,) * 6                                           # x, wq, wk, wv, wo, dy
    grads = (fake, fake, fake, fake)                             # dwq, dwk, dwv, dwo
    assert lh.lh_layer_backward(*head, fake, saved, fake, "f32", *grads, B, H, N, dm, d, L, p, k, "f32", fake,
                                bws - 1) == 4
    assert lh.lh_layer_backward(*head, fake, saved - 1, fake, "f32", *grads, B, H, N, dm, d, L, p, k, "f32", fake,
                                bws) == 4
    assert lh.lh_layer_backward(*head, fake, saved, fake, "f32", None, fake, fake, fake, B, H, N, dm, d, L, p, k,
                                "f32", fake, bws) == 1
    assert lh.lh_layer_backward(*head, fake, saved, fake + 4, "f32", *grads, B, H, N, dm, d, L, p, k, "f32", fake,
                                bws) == 1
    assert lh.library().lh_layer_backward(*head, fake, saved, fake, 9, *grads, B, H, N, dm, d, L, p, k, 0, fake, bws,
                                          None) == 1


def test_binding_refuses_host_tensors(lh):
    """The convenience wrappers refuse host tensors before anything reaches the
    library (a host pointer handed to a kernel would fault the GPU)."""
    import torch
    q = torch.zeros((1, 2, 1024, 64))
    with pytest.raises(ValueError, match="device"):
        lh.forward(q, q, q, 3, 4, 64)
    with pytest.raises(ValueError, match="device"):
        lh.backward(q, q, q, q, torch.zeros(16, dtype=torch.uint8), lh.Plan(1, 2, 1024, 64, 3, 4, 64, "f32"))
    x = torch.zeros((1, 1024, 128))
    w = torch.zeros((128, 128))
    with pytest.raises(ValueError, match="device"):
        lh.layer_forward(x, w, w, w, w, 2, 3, 4, 64)


def test_noalloc_backward_refuses_beyond_its_array(lh):
    """The no-allocation dense backward bounds its rows by its fixed array
    (8 bytes per row in bf16, 4 in fp32, 32 MiB): larger shapes fail validation
    on the host, before any device call."""
    fake = 1 << 20                     # aligned, never dereferenced
    args = [fake] * 9
    limit_bf16, limit_f32 = (32 << 20) // 8, (32 << 20) // 4
    assert lh.lh_attention_backward_noalloc(*args, 8, limit_bf16 // 8 + 64, 128, "bf16") == 4
    assert "scratch" in lh.lh_last_error()
    assert lh.lh_attention_backward_noalloc(*args, 1, limit_f32 + 1, 64, "f32") == 4
    # other validation as the workspace variant: S not a multiple of 64 in bf16, bad d, null pointers
    assert lh.lh_attention_backward_noalloc(*args, 1, 100, 128, "bf16") == 3
    assert lh.lh_attention_backward_noalloc(*args, 1, 128, 96, "bf16") == 3
    assert lh.lh_attention_backward_noalloc(None, *args[1:], 1, 128, 128, "bf16") == 1
