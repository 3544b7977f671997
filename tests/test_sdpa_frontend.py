"""The SDPA-pattern front end on the CPU: which graphs it rewrites, which it
leaves alone and why (shapes propagate on meta tensors; nothing runs)."""

import math

import pytest
import torch
import torch.nn.functional as F

from streaming_attention_amd import sdpa_frontend as fe


def _t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


class Explicit(torch.nn.Module):
    def forward(self, q, k, v):
        s = torch.matmul(q, k.transpose(-2, -1)) / math.sqrt(q.shape[-1])
        return torch.softmax(s, dim=-1) @ v


class ExplicitScaledQ(torch.nn.Module):
    def forward(self, q, k, v):
        s = (q * 0.125) @ k.transpose(2, 3)
        return torch.matmul(F.softmax(s, dim=3), v)


class ExplicitUnscaled(torch.nn.Module):
    def forward(self, q, k, v):
        return (q @ k.mT).softmax(dim=-1) @ v


class Sdpa(torch.nn.Module):
    def __init__(self, **kw):
        super().__init__()
        self.kw = kw

    def forward(self, q, k, v):
        return F.scaled_dot_product_attention(q, k, v, **self.kw) * 2.0


class NotAttention(torch.nn.Module):
    def forward(self, q, k, v):
        a = torch.softmax(q @ k.transpose(-2, -1), dim=2) @ v      # softmax over the query axis
        b = torch.softmax(q @ k, dim=-1)                          # no transpose of K
        return a, b


class BufferCausal(torch.nn.Module):
    """Causal mask as a lower-triangular module buffer sliced to the sequence length."""

    def __init__(self, n=512):
        super().__init__()
        self.register_buffer("tri", torch.tril(torch.ones(n, n)).view(1, 1, n, n))

    def forward(self, q, k, v):
        T = q.size(2)
        att = (q @ k.transpose(-2, -1)) * (1.0 / math.sqrt(k.size(-1)))
        att = att.masked_fill(self.tri[:, :, :T, :T] == 0, float("-inf"))
        return F.softmax(att, dim=-1) @ v


class BottomRightCausal(torch.nn.Module):
    """Causal mask built in forward, aligned so that the last query sees every key."""

    def forward(self, q, k, v):
        Sq, Skv = q.shape[2], k.shape[2]
        hide = q.new_ones(Sq, Skv, dtype=torch.bool).triu(Skv - Sq + 1)
        s = torch.matmul(q, k.transpose(-2, -1)).masked_fill(hide, float("-inf"))
        return torch.softmax(s * 0.125, dim=-1) @ v


class AdditiveMask(torch.nn.Module):
    """An added bias buffer (0 where visible, -inf where hidden), after the scale."""

    def __init__(self, bias):
        super().__init__()
        self.register_buffer("bias", bias)

    def forward(self, q, k, v):
        s = q @ k.transpose(-2, -1) / 8.0
        return torch.softmax(s + self.bias, dim=-1) @ v


class DataMask(torch.nn.Module):
    def forward(self, q, k, v):
        s = (q @ k.transpose(-2, -1)).masked_fill(k.sum(-1, keepdim=True).transpose(-2, -1) > 0, float("-inf"))
        return torch.softmax(s, dim=-1) @ v


def _additive(Sq, Skv, diag):
    b = torch.zeros(Sq, Skv)
    return b.masked_fill(torch.ones(Sq, Skv, dtype=torch.bool).triu(diag), float("-inf"))


def test_causal_masks_in_the_chain_are_recognised():
    q = _t(1, 2, 100, 64)
    gm, rep = fe.rewrite(BufferCausal(), q, q, q)
    (call,) = _calls(gm)
    assert call.kwargs == {"causal": True, "scale": pytest.approx(0.125), "lengths": (100, 100)}
    assert not [n for n in gm.graph.nodes if n.op == "get_attr"]          # the mask buffer is no longer read
    kv = _t(1, 2, 300, 64)
    gm, rep = fe.rewrite(BottomRightCausal(), q, kv, kv)
    (call,) = _calls(gm)
    assert call.kwargs == {"causal": True, "scale": 0.125, "align": "bottom_right", "lengths": (100, 300)}
    gm, rep = fe.rewrite(AdditiveMask(_additive(100, 300, 1)), q, kv, kv)
    (call,) = _calls(gm)
    assert call.kwargs == {"causal": True, "scale": 0.125, "lengths": (100, 300)}   # top-left
    gm, rep = fe.rewrite(AdditiveMask(_additive(100, 300, 201).view(1, 1, 100, 300)), q, kv, kv)
    (call,) = _calls(gm)
    assert call.kwargs["align"] == "bottom_right"


@pytest.mark.parametrize("mod,why", [
    (AdditiveMask(_additive(100, 300, 2)), "not causal"),                     # off by one diagonal
    (AdditiveMask(_additive(100, 300, 1) + torch.linspace(-1, 0, 300)), "other than 0 and -inf"),
    (AdditiveMask(torch.stack([_additive(100, 300, 1), _additive(100, 300, 201)]).view(1, 2, 100, 300)),
     "not causal"),                                                           # differs between heads
    (DataMask(), "depends on"),
])
def test_other_masks_are_left_alone(mod, why):
    q, kv = _t(1, 2, 100, 64), _t(1, 2, 300, 64)
    gm, rep = fe.rewrite(mod, q, kv, kv)
    assert not _calls(gm)
    assert len(rep.skipped) == 1 and why in rep.skipped[0][1], rep.skipped


def test_masked_fill_with_a_finite_value_is_not_matched():
    class Finite(torch.nn.Module):
        def forward(self, q, k, v):
            hide = q.new_ones(q.shape[2], k.shape[2], dtype=torch.bool).triu(1)
            return torch.softmax((q @ k.transpose(-2, -1)).masked_fill(hide, -1e4), dim=-1) @ v

    q = _t(1, 2, 64, 64)
    gm, rep = fe.rewrite(Finite(), q, q, q)
    assert not _calls(gm) and not rep.rewritten and not rep.skipped


class SoftmaxModule(torch.nn.Module):
    """The softmax as an nn.Softmax submodule (a leaf of the trace)."""

    def __init__(self):
        super().__init__()
        self.softmax = torch.nn.Softmax(dim=-1)

    def forward(self, q, k, v):
        return torch.matmul(self.softmax(torch.matmul(q, k.transpose(-1, -2)) * 0.125), v)


def test_softmax_submodule_is_matched():
    q = _t(1, 2, 48, 64)
    gm, rep = fe.rewrite(SoftmaxModule(), q, q, q)
    (call,) = _calls(gm)
    assert call.kwargs == {"causal": False, "scale": 0.125}
    assert not [n for n in gm.graph.nodes if n.op == "call_module"]


def _repeat_kv(x, n_rep):
    """Grouped-query K / V repeated along the head dim (expand + reshape)."""
    b, h, s_, d = x.shape
    return x[:, :, None, :, :].expand(b, h, n_rep, s_, d).reshape(b, h * n_rep, s_, d)


class LlamaStyle(torch.nn.Module):
    """Eager grouped-query attention as transformer code often writes it: K / V
    repeated per query head, fp32 softmax cast back, dropout that is off."""

    def __init__(self, n_rep, causal_len=None):
        super().__init__()
        self.n_rep = n_rep
        self.drop = torch.nn.Dropout(0.1)
        if causal_len:
            self.register_buffer("tri", torch.tril(torch.ones(causal_len, causal_len, dtype=torch.bool)))
        else:
            self.tri = None

    def forward(self, q, k, v):
        k = _repeat_kv(k, self.n_rep)
        v = _repeat_kv(v, self.n_rep)
        w = torch.matmul(q, k.transpose(2, 3)) * (q.shape[-1] ** -0.5)
        if self.tri is not None:
            T = q.shape[2]
            w = w.masked_fill(~self.tri[:T, :T], float("-inf"))
        w = F.softmax(w, dim=-1, dtype=torch.float32).to(q.dtype)
        w = F.dropout(w, p=0.1, training=False)
        w = self.drop(w)
        return torch.matmul(w, v).transpose(1, 2).contiguous()


class RepeatInterleave(torch.nn.Module):
    def forward(self, q, k, v):
        k = k.repeat_interleave(4, dim=1)
        v = torch.repeat_interleave(v, 4, dim=1)
        return torch.softmax(q @ k.transpose(-2, -1) * 0.125, dim=-1) @ v


@pytest.mark.parametrize("mod,causal", [(LlamaStyle(4).eval(), False), (LlamaStyle(4, 256).eval(), True),
                                        (RepeatInterleave(), False)])
def test_repeated_kv_heads_are_read_once(mod, causal):
    q, kv = _t(1, 8, 96, 64), _t(1, 2, 96, 64)
    gm, rep = fe.rewrite(mod, q, kv, kv)
    (call,) = _calls(gm)
    assert [a.name for a in call.args] == ["q", "k", "v"]          # the unrepeated K and V
    assert call.kwargs["causal"] is causal and call.kwargs["scale"] == pytest.approx(0.125)
    left = {getattr(n.target, "__name__", str(n.target)) for n in gm.graph.nodes if n.op in ("call_method",
                                                                                             "call_function")}
    assert not left & {"expand", "reshape", "repeat_interleave", "softmax", "dropout", "matmul"}, left


def test_dropout_in_training_is_not_passed_over():
    mod = LlamaStyle(4).train()
    q, kv = _t(1, 8, 32, 64), _t(1, 2, 32, 64)
    gm, rep = fe.rewrite(mod, q, kv, kv)
    assert not _calls(gm) and not rep.rewritten


class SdpaMask(torch.nn.Module):
    """SDPA with an explicit attn_mask buffer (bool: True = keep; float: added)."""

    def __init__(self, mask, **kw):
        super().__init__()
        self.register_buffer("mask", mask)
        self.kw = kw

    def forward(self, q, k, v):
        return F.scaled_dot_product_attention(q, k, v, attn_mask=self.mask, **self.kw)


class SdpaMaskInput(torch.nn.Module):
    def forward(self, q, k, v, m):
        return F.scaled_dot_product_attention(q, k, v, attn_mask=m)


def test_sdpa_causal_attn_masks_are_recognised():
    q, kv = _t(1, 2, 100, 64), _t(1, 2, 300, 64)
    keep = torch.ones(100, 300, dtype=torch.bool).tril()                      # top-left
    gm, rep = fe.rewrite(SdpaMask(keep), q, kv, kv)
    (call,) = _calls(gm)
    assert call.kwargs == {"causal": True, "scale": pytest.approx(0.125), "lengths": (100, 300)}
    gm, rep = fe.rewrite(SdpaMask(_additive(100, 300, 201), scale=0.5), q, kv, kv)   # bottom-right, float
    (call,) = _calls(gm)
    assert call.kwargs == {"causal": True, "scale": 0.5, "align": "bottom_right", "lengths": (100, 300)}


@pytest.mark.parametrize("mod,extra,why", [
    (SdpaMask(torch.ones(100, 300, dtype=torch.bool).tril(1)), [], "not causal"),
    (SdpaMaskInput(), [torch.ones(100, 300, dtype=torch.bool)], "depends on"),
])
def test_other_sdpa_masks_are_left_alone(mod, extra, why):
    q, kv = _t(1, 2, 100, 64), _t(1, 2, 300, 64)
    gm, rep = fe.rewrite(mod, q, kv, kv, *extra)
    assert not _calls(gm)
    assert len(rep.skipped) == 1 and why in rep.skipped[0][1], rep.skipped


class TwoBlocks(torch.nn.Module):
    """Two attention blocks in one graph: a causal SDPA call feeding an explicit chain."""

    def forward(self, q, k, v):
        h = F.scaled_dot_product_attention(q, k, v, is_causal=True)
        return torch.softmax(h @ k.transpose(-2, -1) * 0.125, dim=-1) @ v + h


def test_every_match_in_a_graph_is_rewritten():
    q = _t(1, 2, 64, 64)
    gm, rep = fe.rewrite(TwoBlocks(), q, q, q)
    calls = _calls(gm)
    assert len(calls) == 2 and len(rep.rewritten) == 2
    assert sorted(c.kwargs["causal"] for c in calls) == [False, True]
    assert calls[1].args[0] is calls[0] or calls[0].args[0] is calls[1]     # the second block reads the first


class WeightsReturned(torch.nn.Module):
    """The attention weights are an output too: the chain must stay as written."""

    def forward(self, q, k, v):
        w = torch.softmax(q @ k.transpose(-2, -1) * 0.125, dim=-1)
        return w @ v, w


class ScaledQShared(torch.nn.Module):
    """Q is scaled once and the scaled Q is also used elsewhere."""

    def forward(self, q, k, v):
        qs = q * 0.125
        return torch.softmax(qs @ k.transpose(-2, -1), dim=-1) @ v, qs.sum()


def test_weights_used_elsewhere_keep_the_chain():
    q = _t(1, 2, 32, 64)
    gm, rep = fe.rewrite(WeightsReturned(), q, q, q)
    assert not _calls(gm) and not rep.rewritten


def test_a_scaled_q_with_other_users_stays_for_them():
    q = _t(1, 2, 32, 64)
    gm, rep = fe.rewrite(ScaledQShared(), q, q, q)
    (call,) = _calls(gm)
    assert call.args[0].name == "q" and call.kwargs["scale"] == 0.125
    assert any(n.op == "call_method" and n.target == "sum" for n in gm.graph.nodes)


def test_one_broadcast_kv_head_is_legal():
    gm, rep = fe.rewrite(Explicit(), _t(1, 8, 32, 64), _t(1, 1, 32, 64), _t(1, 1, 32, 64))
    assert len(_calls(gm)) == 1 and not rep.skipped


def _calls(gm):
    return [n for n in gm.graph.nodes if n.op == "call_function" and n.target is fe.fused_attention]


@pytest.mark.parametrize("mod,scale", [(Explicit(), 1 / math.sqrt(128)), (ExplicitScaledQ(), 0.125),
                                       (ExplicitUnscaled(), 1.0)])
def test_explicit_chains_are_rewritten(mod, scale):
    q = _t(2, 4, 64, 128)
    gm, rep = fe.rewrite(mod, q, q, q)
    (call,) = _calls(gm)
    assert call.kwargs == {"causal": False, "scale": pytest.approx(scale)}
    names = {getattr(n.target, "__name__", str(n.target)) for n in gm.graph.nodes if n.op != "placeholder"}
    assert "softmax" not in names and "matmul" not in names
    assert len(rep.rewritten) == 1 and not rep.skipped


def test_sdpa_calls_are_rewritten_with_their_flags():
    q, k = _t(1, 8, 64, 128), _t(1, 2, 64, 128)
    gm, rep = fe.rewrite(Sdpa(is_causal=True, enable_gqa=True), q, k, k)
    (call,) = _calls(gm)
    assert call.kwargs == {"causal": True, "scale": pytest.approx(1 / math.sqrt(128))}
    gm, _ = fe.rewrite(Sdpa(scale=0.5), q, q, q)
    (call,) = _calls(gm)
    assert call.kwargs == {"causal": False, "scale": 0.5}


@pytest.mark.parametrize("mod,shapes,dtype,why", [
    (Explicit(), [(1, 2, 16, 96)] * 3, torch.bfloat16, "head dim"),
    (Explicit(), [(1, 2, 16, 64)] * 3, torch.float16, "dtype"),
    (Explicit(), [(2, 16, 64)] * 3, torch.bfloat16, "[B, H, S, d]"),
    (Sdpa(is_causal=True), [(1, 2, 32, 64), (1, 2, 16, 64), (1, 2, 16, 64)], torch.bfloat16, "more queries"),
    (Explicit(), [(1, 2, 16, 128), (1, 2, 16, 128), (1, 2, 16, 64)], torch.bfloat16, "K / V shapes"),
])
def test_illegal_matches_are_left_alone(mod, shapes, dtype, why):
    args = [_t(*s, dtype=dtype) for s in shapes]
    gm, rep = fe.rewrite(mod, *args)
    assert not _calls(gm)
    assert len(rep.skipped) == 1 and why in rep.skipped[0][1]


class SdpaShapeFlags(torch.nn.Module):
    """SDPA flags computed from shapes: causal only when there is more than
    one query, the scale from the head dim."""

    def forward(self, q, k, v):
        return F.scaled_dot_product_attention(q, k, v, is_causal=q.shape[2] > 1, scale=q.shape[-1] ** -0.5)


class SdpaFlagInput(torch.nn.Module):
    """The causal flag is an input of the graph: its value at rewrite time says
    nothing about later calls."""

    def forward(self, q, k, v, causal):
        return F.scaled_dot_product_attention(q, k, v, is_causal=causal)


def test_sdpa_flags_computed_from_shapes_take_their_values():
    """is_causal = (Sq > 1) is False for one query: the rewrite must not be
    causal (a causal top-left call would see only key 0)."""
    q, kv = _t(1, 2, 1, 64), _t(1, 2, 40, 64)
    gm, rep = fe.rewrite(SdpaShapeFlags(), q, kv, kv)
    (call,) = _calls(gm)
    assert call.kwargs == {"causal": False, "scale": pytest.approx(0.125)}
    q = _t(1, 2, 40, 128)
    gm, rep = fe.rewrite(SdpaShapeFlags(), q, q, q)
    (call,) = _calls(gm)
    assert call.kwargs == {"causal": True, "scale": pytest.approx(1 / math.sqrt(128))}


def test_sdpa_flags_that_are_inputs_are_left_alone():
    q = _t(1, 2, 8, 64)
    gm, rep = fe.rewrite(SdpaFlagInput(), q, q, q, True)
    assert not _calls(gm)
    assert len(rep.skipped) == 1 and "is_causal not a constant" in rep.skipped[0][1], rep.skipped


class SlidingWindow(torch.nn.Module):
    """A causal mask limited to the last `window` keys: causal-looking while
    every sequence is shorter than the window."""

    def __init__(self, window):
        super().__init__()
        self.window = window

    def forward(self, q, k, v):
        T = q.shape[2]
        ones = q.new_ones(T, T, dtype=torch.bool)
        hide = ones.triu(1) | ones.tril(-self.window)
        s = (q @ k.transpose(-2, -1)).masked_fill(hide, float("-inf"))
        return torch.softmax(s * 0.125, dim=-1) @ v


def test_a_window_mask_is_only_trusted_at_the_lengths_it_was_checked():
    q = _t(1, 2, 64, 64)
    gm, rep = fe.rewrite(SlidingWindow(100), q, q, q)          # at T = 64 the window hides nothing
    (call,) = _calls(gm)
    assert call.kwargs["lengths"] == (64, 64)
    big = _t(1, 2, 200, 64)
    with pytest.raises(ValueError, match="checked at"):
        gm(big, big, big)                                      # refused before anything runs
    gm, rep = fe.rewrite(SlidingWindow(100), big, big, big)    # at T = 200 the window shows
    assert not _calls(gm)
    assert len(rep.skipped) == 1 and "not causal" in rep.skipped[0][1]


def test_masked_or_dropout_sdpa_and_other_softmaxes_are_not_matched():
    q = _t(1, 2, 16, 64)
    gm, rep = fe.rewrite(Sdpa(attn_mask=None, dropout_p=0.1), q, q, q)
    assert not _calls(gm) and not rep.rewritten
    q = _t(1, 2, 16, 16)
    gm, rep = fe.rewrite(NotAttention(), q, q, q)
    assert not _calls(gm) and not rep.rewritten and not rep.skipped


# ---- GPU: the rewritten modules against the float64 oracle -------------------------------------------------
# The original modules never run on the GPU: only their rewritten graphs, from which every matmul and softmax
# of the matched region has been removed (no batched bf16 product with a transposed operand runs).

def _gpu_inputs(seed, shapes, dtype):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return [torch.randn(s, generator=g, device="cuda").to(dtype) for s in shapes]


def _run_rewritten(mod, args):
    return _run_rewritten_n(mod, args, 1)


def _run_rewritten_n(mod, args, n_calls):
    gm, rep = fe.rewrite(mod, *args)
    assert len(_calls(gm)) == n_calls and not rep.skipped
    left = {getattr(n.target, "__name__", str(n.target)) for n in gm.graph.nodes if n.op != "placeholder"}
    assert not left & {"matmul", "bmm", "softmax", "scaled_dot_product_attention"}, left
    out = gm(*args)
    torch.cuda.synchronize()
    return out


@pytest.mark.gpu
@pytest.mark.parametrize("mod,shapes,dtype,scale", [
    (Explicit(), [(1, 4, 200, 128)] * 3, torch.bfloat16, 1 / math.sqrt(128)),
    (ExplicitScaledQ(), [(2, 2, 130, 64)] * 3, torch.float32, 0.125),
    (Explicit(), [(1, 8, 96, 64), (1, 1, 300, 64), (1, 1, 300, 64)], torch.bfloat16, 1 / 8.0),
])
def test_rewritten_explicit_chain_matches_oracle(mod, shapes, dtype, scale):
    import oracle
    from parity import assert_o, f64

    q, k, v = _gpu_inputs(11, shapes, dtype)
    o = _run_rewritten(mod, [q, k, v])
    O_ref, _ = oracle.attention(f64(q), f64(k), f64(v), scale, False)
    assert_o(o, O_ref, "bf16" if dtype == torch.bfloat16 else "f32")


@pytest.mark.gpu
@pytest.mark.parametrize("Sq,Skv,kw", [
    (150, 150, dict(is_causal=True, enable_gqa=True)),
    (100, 300, dict(is_causal=True, enable_gqa=True)),          # top-left causal: the first Sq keys
    (100, 300, dict(scale=0.05, enable_gqa=True)),
])
def test_rewritten_sdpa_matches_oracle(Sq, Skv, kw):
    import oracle
    from parity import assert_o, f64

    q, k, v = _gpu_inputs(12, [(1, 8, Sq, 128), (1, 2, Skv, 128), (1, 2, Skv, 128)], torch.bfloat16)
    o = _run_rewritten(Sdpa(**kw), [q, k, v])
    causal = kw.get("is_causal", False)
    scale = kw.get("scale", 1 / math.sqrt(128))
    n = Sq if causal else Skv       # a top-left causal mask hides every key at or past position Sq
    O_ref, _ = oracle.attention(f64(q), f64(k)[:, :, :n], f64(v)[:, :, :n], scale, causal)
    assert_o(o, 2.0 * O_ref, "bf16")          # the module doubles the attention output


@pytest.mark.gpu
@pytest.mark.parametrize("causal", [False, True])
def test_rewritten_llama_style_gqa_matches_oracle(causal):
    import oracle
    from parity import assert_o, f64

    mod = LlamaStyle(4, 512 if causal else None).eval().cuda()
    q, k, v = _gpu_inputs(14, [(2, 16, 200, 128), (2, 4, 200, 128), (2, 4, 200, 128)], torch.bfloat16)
    o = _run_rewritten(mod, [q, k, v])
    O_ref, _ = oracle.attention(f64(q), f64(k), f64(v), 128 ** -0.5, causal)
    assert_o(o, O_ref.transpose(0, 2, 1, 3), "bf16")


@pytest.mark.gpu
def test_rewritten_two_block_graph_matches_oracle():
    import oracle
    from parity import assert_o, f64

    q, k, v = _gpu_inputs(16, [(1, 4, 96, 64)] * 3, torch.bfloat16)
    out = _run_rewritten_n(TwoBlocks(), [q, k, v], 2)
    H, _ = oracle.attention(f64(q), f64(k), f64(v), 0.125, True)
    h = torch.tensor(H, dtype=torch.float32).to(torch.bfloat16)       # the first block's output as the kernel stores it
    O2, _ = oracle.attention(f64(h), f64(k), f64(v), 0.125, False)
    assert_o(out, O2 + f64(h), "bf16")


@pytest.mark.gpu
def test_rewritten_sdpa_with_causal_attn_mask_matches_oracle():
    import oracle
    from parity import assert_o, f64

    mod = SdpaMask(torch.ones(100, 300, dtype=torch.bool).tril(200), enable_gqa=True).cuda()   # bottom-right
    q, k, v = _gpu_inputs(15, [(2, 8, 100, 128), (2, 2, 300, 128), (2, 2, 300, 128)], torch.bfloat16)
    o = _run_rewritten(mod, [q, k, v])
    O_ref, _ = oracle.attention(f64(q), f64(k), f64(v), 128 ** -0.5, True)
    assert_o(o, O_ref, "bf16")


@pytest.mark.gpu
@pytest.mark.parametrize("mod,Sq,Skv,top_left", [
    (BufferCausal(), 200, 200, True),
    (BottomRightCausal(), 100, 300, False),
    (AdditiveMask(_additive(100, 300, 1)), 100, 300, True),
])
def test_rewritten_masked_chain_matches_oracle(mod, Sq, Skv, top_left):
    import oracle
    from parity import assert_o, f64

    mod = mod.cuda()
    q, k, v = _gpu_inputs(13, [(2, 4, Sq, 64), (2, 4, Skv, 64), (2, 4, Skv, 64)], torch.bfloat16)
    o = _run_rewritten(mod, [q, k, v])
    n = Sq if top_left else Skv
    O_ref, _ = oracle.attention(f64(q), f64(k)[:, :, :n], f64(v)[:, :, :n], 0.125, True)
    assert_o(o, O_ref, "bf16")
