"""SDPA-pattern front end: find scaled-dot-product attention in a torch.fx
graph and route it to the library's fused kernel.

The three steps follow "AI Compiler pipeline stages" (its pattern matching,
legality checking and rewrite stages) and "MCIR Minimal Implementation
Design" section 9 (the score product, an optional mask, the softmax and the
product with V are recognised as one attention pattern in the operator graph
and lowered to a streaming region):

* pattern: ``softmax(mask(scale * (Q @ K^T)), dim=-1) @ V`` written out (the
  scale as a constant multiply or divide of the scores, or of Q, before or
  after the mask; the mask optional), and calls of
  ``torch.nn.functional.scaled_dot_product_attention`` without dropout
  (``is_causal``, or an ``attn_mask`` that is causal).  A mask is
  ``masked_fill(M, -inf)``, an added bias of 0 / -inf, or SDPA's boolean
  (keep) or float (bias) ``attn_mask``, computed from constants, module
  buffers and shapes only.  Its values are evaluated once at rewrite time
  and accepted when they are exactly a causal mask (the causal attention
  pattern of "AI Compiler pipeline stages", Pattern Matching), aligned
  top-left (query t sees keys 0..t) or bottom-right (query t sees keys
  0..Skv-Sq+t); the rewritten call then refuses other lengths, since a
  window or padding mask can look causal at one length only.  Flags of an
  SDPA call computed from shapes (``is_causal=q.shape[2] > 1``) count as
  constants; flags that depend on data leave the call alone.  Between the softmax and the P V product, casts,
  ``contiguous`` and dropout that is off (p = 0, or not training at rewrite
  time: the rewritten graph is for inference) are passed over.  K and V
  repeated along the head dim for grouped-query attention
  (``repeat_interleave(G, dim=1)``, or the unsqueeze-expand-reshape idiom)
  are matched back to the unrepeated tensors, which the kernel reads once
  per KV head;
* legality, from shapes and dtypes propagated on meta tensors: 4-D
  ``[B, H, S, d]`` operands of one dtype (bf16 or fp32), d 64 or 128, query
  heads a multiple of KV heads (one KV head, ``enable_gqa``, or repeated
  K / V), and for causal attention at most as many queries as keys;
* rewrite: the matched nodes are replaced by one call of
  :func:`fused_attention`, which runs ``attn_prefill`` (or split-KV +
  merge) through the binding.

Graph edits only: nothing here computes attention.  Unmatched or illegal
subgraphs are left as they are, and the report says why.
"""

from __future__ import annotations

import copy
import dataclasses
import math
import operator

import torch
import torch.fx as fx
from torch.fx.passes.shape_prop import ShapeProp

from . import _binding

_SOFTMAX = {torch.softmax, torch.nn.functional.softmax}
_MATMUL = {torch.matmul, operator.matmul}
_SDPA = torch.nn.functional.scaled_dot_product_attention


def fused_attention(q, k, v, causal: bool, scale: float, align: str = "top_left", lengths=None):
    """The rewritten region: softmax(scale Q K^T [+ causal mask]) V on the GPU.

    SDPA's ``is_causal`` mask is top-left aligned (query t sees keys 0..t); the
    kernel aligns bottom-right (the last query sees every key), so with fewer
    queries than keys a top-left mask passes only the first Sq keys -- the only
    ones any query can see.

    ``lengths = (Sq, Skv)``: the region's mask was recognised from its values
    at these lengths only (a window or padding mask can look causal at one
    length and not at another), so other lengths are refused.
    """
    if lengths is not None and (q.shape[2], k.shape[2]) != tuple(lengths):
        raise ValueError(f"this attention region's mask was checked at (Sq, Skv) = {tuple(lengths)}; "
                         f"called with {(q.shape[2], k.shape[2])}: rewrite the module at these lengths")
    if causal and align == "top_left" and q.shape[2] < k.shape[2]:
        k = k[:, :, :q.shape[2]]
        v = v[:, :, :q.shape[2]]
    return _binding.prefill(q.contiguous(), k.contiguous(), v.contiguous(), causal=causal, scale=float(scale),
                            return_lse=False)


@dataclasses.dataclass
class Match:
    q: fx.Node
    k: fx.Node
    v: fx.Node
    scale: float | None      # None: 1 / sqrt(d)
    causal: bool
    out: fx.Node             # node whose uses the fused call takes over
    kind: str                # "explicit" or "sdpa"
    gqa: bool = False        # SDPA's enable_gqa, or K / V repeats matched away
    align: str = "top_left"  # causal mask alignment: "top_left" or "bottom_right"
    error: str | None = None        # why the region cannot be rewritten (its mask, a non-constant argument)
    mask_lengths: tuple | None = None   # (Sq, Skv) at which a mask's values were checked


def _const(x):
    """The number x stands for: a literal, or a node whose value shape
    propagation found to be a plain number (e.g. ``math.sqrt(q.shape[-1])``)."""
    if isinstance(x, fx.Node):
        x = x.meta.get("scalar_value")
    return x if isinstance(x, (int, float)) and not isinstance(x, bool) else None


_UNKNOWN = object()


def _static(x):
    """The value x stands for: a literal, or a node whose value shape
    propagation found to depend on shapes only (numbers, bools, sizes);
    ``_UNKNOWN`` for a node whose value depends on an input's data."""
    if isinstance(x, fx.Node):
        return x.meta.get("static_value", _UNKNOWN)
    return x


def _is_static(x) -> bool:
    if isinstance(x, (int, float, bool, torch.dtype)):
        return True
    return isinstance(x, (tuple, list, torch.Size)) and all(_is_static(e) for e in x)


class _ShapeAndScalarProp(ShapeProp):
    """ShapeProp that also keeps the value of every node that evaluates to a
    plain number or a tuple of them (sizes): on meta tensors such values
    depend on shapes only, so scales and slice bounds computed from shapes are
    known constants."""

    def run_node(self, n):
        result = super().run_node(n)
        if n.op == "placeholder":                 # an input's value is the caller's, not a constant
            return result
        if isinstance(result, torch.device):      # masks are evaluated on the CPU
            n.meta["static_value"] = torch.device("cpu")
        if _is_static(result):
            n.meta["static_value"] = result
            if isinstance(result, (int, float)) and not isinstance(result, bool):
                n.meta["scalar_value"] = result
        return result


def _single_user(n: fx.Node) -> bool:
    return len(n.users) == 1


def _is_last2_transpose(n) -> fx.Node | None:
    """K if n is K^T over the last two dims, else None."""
    if not isinstance(n, fx.Node):
        return None
    if n.op == "call_method" and n.target == "transpose" and len(n.args) == 3:
        if {n.args[1], n.args[2]} in ({-2, -1}, {2, 3}):
            return n.args[0]
    if n.op == "call_function" and n.target is torch.transpose and len(n.args) == 3:
        if {n.args[1], n.args[2]} in ({-2, -1}, {2, 3}):
            return n.args[0]
    if n.op == "call_function" and n.target is getattr and n.args[1] == "mT":
        return n.args[0]
    return None


def _is_matmul(n) -> bool:
    return isinstance(n, fx.Node) and ((n.op == "call_function" and n.target in _MATMUL)
                                       or (n.op == "call_method" and n.target == "matmul"))


def _softmax_last_dim(n, gm=None) -> fx.Node | None:
    """The scores node if n is a softmax over the last dim (function, method
    or an ``nn.Softmax`` submodule), else None."""
    if not isinstance(n, fx.Node):
        return None
    dim = None
    if n.op == "call_function" and n.target in _SOFTMAX:
        dim = n.kwargs.get("dim", n.args[1] if len(n.args) > 1 else None)
    elif n.op == "call_method" and n.target == "softmax":
        dim = n.kwargs.get("dim", n.args[1] if len(n.args) > 1 else None)
    elif n.op == "call_module" and gm is not None and isinstance(_fetch_attr(gm, n.target), torch.nn.Softmax):
        dim = _fetch_attr(gm, n.target).dim
    else:
        return None
    return n.args[0] if dim in (-1, 3) else None


def _strip_scale(n):
    """(inner, factor) for n = inner * c, c * inner or inner / c; else (n, 1)."""
    if isinstance(n, fx.Node) and n.op == "call_function":
        if n.target in (operator.mul, torch.mul):
            a, b = n.args[0], n.args[1]
            if _const(b) is not None:
                return a, float(_const(b))
            if _const(a) is not None:
                return b, float(_const(a))
        if n.target in (operator.truediv, torch.div) and _const(n.args[1]) not in (None, 0):
            return n.args[0], 1.0 / float(_const(n.args[1]))
    return n, 1.0


_MAX_MASK_ELEMS = 1 << 26   # masks evaluated at rewrite time are at most this large


_SHAPE_ONLY_METHODS = {"new_ones", "new_zeros", "new_full"}


def _fetch_attr(gm, target: str):
    obj = gm
    for part in target.split("."):
        obj = getattr(obj, part)
    return obj


def _evaluate(gm, n, memo):
    """Value of node n from constants, module attributes and static values
    only; raises LookupError when it depends on an input's data."""
    if not isinstance(n, fx.Node):
        if isinstance(n, (tuple, list)):
            return type(n)(_evaluate(gm, e, memo) for e in n)
        if isinstance(n, slice):
            return slice(_evaluate(gm, n.start, memo), _evaluate(gm, n.stop, memo), _evaluate(gm, n.step, memo))
        if isinstance(n, dict):
            return {k: _evaluate(gm, e, memo) for k, e in n.items()}
        return n
    if n in memo:
        return memo[n]
    if "static_value" in n.meta:
        val = n.meta["static_value"]
    elif n.op == "get_attr":
        val = _fetch_attr(gm, n.target)
        if isinstance(val, torch.Tensor):
            val = val.detach().cpu()
    elif n.op in ("call_function", "call_method"):
        tm = n.meta.get("tensor_meta")
        if tm is not None and hasattr(tm, "shape") and math.prod(tm.shape) > _MAX_MASK_ELEMS:
            raise LookupError("mask too large to check")
        if n.op == "call_method" and n.target in _SHAPE_ONLY_METHODS and isinstance(n.args[0], fx.Node):
            # x.new_ones(...) and the like read only x's dtype: a CPU stand-in of that dtype will do
            tm0 = n.args[0].meta.get("tensor_meta")
            if tm0 is None:
                raise LookupError(f"no dtype for {n.args[0].name}")
            args = (torch.empty(0, dtype=tm0.dtype),) + tuple(_evaluate(gm, n.args[1:], memo))
        else:
            args = _evaluate(gm, n.args, memo)
        kwargs = _evaluate(gm, n.kwargs, memo)
        if n.op == "call_function":
            val = n.target(*args, **kwargs)
        else:
            val = getattr(args[0], n.target)(*args[1:], **kwargs)
    else:
        raise LookupError(f"mask depends on {n.op} {n.name}")
    memo[n] = val
    return val


def _causal_alignment(masked: torch.Tensor, Sq: int, Skv: int) -> str | None:
    """'top_left' / 'bottom_right' if the boolean ``masked`` (True = key hidden),
    broadcast over any leading dims, is exactly that causal mask; else None."""
    if masked.dim() < 2 or masked.shape[-2] not in (1, Sq) or masked.shape[-1] not in (1, Skv):
        return None
    m = masked.reshape(-1, masked.shape[-2], masked.shape[-1])
    if not bool((m == m[:1]).all()):
        return None
    m = m[0].expand(Sq, Skv)
    i = torch.arange(Sq).unsqueeze(1)
    j = torch.arange(Skv).unsqueeze(0)
    if torch.equal(m, j > i):
        return "top_left"
    if torch.equal(m, j > i + (Skv - Sq)):
        return "bottom_right"
    return None


_NEG_INF_LIKE = -1e30      # fill values at or below this act as -inf after the max subtraction


def _strip_mask(n):
    """(inner, mask node, how) for n = inner.masked_fill(M, v) or inner + bias; else (n, None, None)."""
    if not isinstance(n, fx.Node):
        return n, None, None
    if (n.op == "call_method" and n.target == "masked_fill") or \
            (n.op == "call_function" and n.target is torch.masked_fill):
        value = n.kwargs.get("value", n.args[2] if len(n.args) > 2 else None)
        c = _const(value)
        if c is None or c > _NEG_INF_LIKE:
            return n, None, None
        return n.args[0], n.kwargs.get("mask", n.args[1]), "fill"
    if n.op == "call_function" and n.target in (operator.add, torch.add) and len(n.args) == 2:
        a, b = n.args
        if isinstance(a, fx.Node) and isinstance(b, fx.Node):
            # the bias is the operand that does not come from the score product
            return (a, b, "add") if _is_matmul(_strip_scale(a)[0]) else (b, a, "add")
    return n, None, None


def _mask_alignment(gm, mask_node, how, Sq, Skv) -> tuple[str | None, str | None]:
    """(alignment, None) for a causal mask; (None, reason) otherwise."""
    try:
        val = _evaluate(gm, mask_node, {})
    except LookupError as e:
        return None, str(e)
    except Exception as e:       # the mask subgraph does not evaluate on its own
        return None, f"mask not evaluable ({type(e).__name__})"
    if not isinstance(val, torch.Tensor):
        return None, "mask is not a tensor"
    if how in ("fill", "keep") and val.dtype == torch.bool:
        masked = val if how == "fill" else ~val
    elif how == "fill":
        return None, "masked_fill mask is not boolean"
    else:                          # an added bias (an explicit add, or SDPA's float mask)
        v = val.double()
        masked = v <= _NEG_INF_LIKE
        if not bool(((v == 0) | masked).all()):
            return None, "additive mask holds values other than 0 and -inf"
    align = _causal_alignment(masked, Sq, Skv)
    return (align, None) if align else (None, "mask is not causal")


def _passes_probabilities(n, gm) -> bool:
    """True for a node that hands the probabilities on unchanged up to
    rounding to the P V product's dtype: a cast, ``contiguous``, or dropout
    that is off."""
    if n.op == "call_method" and n.target in ("to", "type", "type_as", "contiguous"):
        return True
    if n.op == "call_function" and n.target is torch.nn.functional.dropout:
        p = n.kwargs.get("p", n.args[1] if len(n.args) > 1 else 0.5)
        training = n.kwargs.get("training", n.args[2] if len(n.args) > 2 else True)
        return p == 0 or training is False
    if n.op == "call_module":
        mod = _fetch_attr(gm, n.target)
        return isinstance(mod, torch.nn.Dropout) and (mod.p == 0 or not mod.training)
    return False


def _unsqueezed_at_2(n) -> fx.Node | None:
    """x if n is x.unsqueeze(2) or x[:, :, None] (x 4-D), else None."""
    if not isinstance(n, fx.Node):
        return None
    if n.op == "call_method" and n.target == "unsqueeze" and len(n.args) == 2 and n.args[1] == 2:
        return n.args[0]
    if n.op == "call_function" and n.target is torch.unsqueeze and len(n.args) == 2 and n.args[1] == 2:
        return n.args[0]
    if n.op == "call_function" and n.target is operator.getitem and isinstance(n.args[1], tuple):
        idx = n.args[1]
        full = slice(None, None, None)
        if len(idx) >= 3 and idx[0] == full and idx[1] == full and idx[2] is None and \
                all(i == full or i is Ellipsis for i in idx[3:]):
            return n.args[0]
    return None


def _strip_kv_repeat(n):
    """(x, G) when n is x with every head repeated G times in a row along dim
    1 -- ``repeat_interleave(G, dim=1)`` or ``x[:, :, None].expand(B, H, G, S,
    d).reshape(B, H * G, S, d)`` -- so that head h of n is head h // G of x;
    else (n, 1).  Shapes come from shape propagation."""
    if not isinstance(n, fx.Node):
        return n, 1
    if (n.op == "call_method" and n.target == "repeat_interleave") or \
            (n.op == "call_function" and n.target is torch.repeat_interleave):
        reps = _const(n.kwargs.get("repeats", n.args[1] if len(n.args) > 1 else None))
        dim = n.kwargs.get("dim", n.args[2] if len(n.args) > 2 else None)
        if isinstance(reps, int) and reps >= 1 and dim in (1, -3):
            return n.args[0], reps
        return n, 1
    if n.op == "call_method" and n.target in ("reshape", "view") and isinstance(n.args[0], fx.Node):
        ex = n.args[0]
        if ex.op != "call_method" or ex.target != "expand":
            return n, 1
        x = _unsqueezed_at_2(ex.args[0])
        tx, te, tn = _meta(x), _meta(ex), _meta(n)
        if x is None or tx is None or te is None or tn is None:
            return n, 1
        xs, es, ns = tuple(tx.shape), tuple(te.shape), tuple(tn.shape)
        if len(xs) == 4 and len(es) == 5 and len(ns) == 4 and es[:2] == xs[:2] and es[3:] == xs[2:] and \
                ns == (xs[0], xs[1] * es[2], xs[2], xs[3]):
            return x, es[2]
    return n, 1


def _explicit_mask(gm, m: Match, mask_node, how: str) -> None:
    """Record on m whether mask_node (used as ``how``) is a causal mask, and
    its alignment; a non-causal mask leaves m illegal with the reason."""
    tq, tk = _meta(m.q), _meta(m.k)
    if tq is None or tk is None or len(tq.shape) < 2 or len(tk.shape) < 2:
        m.error = "no shape information for the mask"
        return
    align, why = _mask_alignment(gm, mask_node, how, tq.shape[-2], tk.shape[-2])
    m.causal = why is None
    m.align, m.error = (align or "top_left"), why
    m.mask_lengths = (int(tq.shape[-2]), int(tk.shape[-2]))


def find_attention(gm: fx.GraphModule) -> list[Match]:
    """Pattern matching: every explicit softmax(mask?(QK^T)) V chain and SDPA call."""
    found = []
    for n in gm.graph.nodes:
        if n.op == "call_function" and n.target is _SDPA:
            args = list(n.args) + [None] * (3 - len(n.args))
            kw = n.kwargs
            # Flags may be graph values computed from shapes (is_causal=q.shape[2] > 1,
            # scale=q.shape[-1] ** -0.5): their static values decide; a flag that
            # depends on an input's data leaves the call as it is.
            dropout = _static(kw.get("dropout_p", n.args[4] if len(n.args) > 4 else 0.0))
            causal = _static(kw.get("is_causal", n.args[5] if len(n.args) > 5 else False))
            scale = _static(kw.get("scale", n.args[6] if len(n.args) > 6 else None))
            gqa = _static(kw.get("enable_gqa", False))
            unknown = [name for name, val in (("dropout_p", dropout), ("is_causal", causal), ("scale", scale),
                                              ("enable_gqa", gqa)) if val is _UNKNOWN]
            if not unknown and dropout not in (0, 0.0):
                continue
            m = Match(args[0], args[1], args[2], None, False, n, "sdpa")
            if unknown:
                m.error = f"{', '.join(unknown)} not a constant at rewrite time"
                found.append(m)
                continue
            if scale is not None and (not isinstance(scale, (int, float)) or isinstance(scale, bool)):
                m.error = f"scale {scale!r} is not a number"
                found.append(m)
                continue
            m.scale = None if scale is None else float(scale)
            m.causal, m.gqa = bool(causal), bool(gqa)
            attn_mask = kw.get("attn_mask", n.args[3] if len(n.args) > 3 else None)
            if attn_mask is not None:   # (PyTorch allows no is_causal with it)
                # SDPA's boolean mask keeps the True entries; a float mask is added to the scores.
                _explicit_mask(gm, m, attn_mask, "keep")
            found.append(m)
            continue
        scores = _softmax_last_dim(n, gm)
        if scores is None or not _single_user(n):
            continue
        probs = n                          # last node before the P V product
        while _single_user(probs) and _passes_probabilities(next(iter(probs.users)), gm):
            probs = next(iter(probs.users))
        if not _single_user(probs):
            continue
        pv = next(iter(probs.users))
        if not _is_matmul(pv) or pv.args[0] is not probs:
            continue
        chain = [scores]                   # nodes between the score product and the softmax
        inner, f1 = _strip_scale(scores)
        if inner is not chain[-1]:
            chain.append(inner)
        inner, mask_node, how = _strip_mask(inner)
        if inner is not chain[-1]:
            chain.append(inner)
        inner, f3 = _strip_scale(inner)
        if inner is not chain[-1]:
            chain.append(inner)
        if not _is_matmul(inner) or not all(isinstance(c, fx.Node) and _single_user(c) for c in chain):
            continue
        qn, f2 = _strip_scale(inner.args[0])
        kn = _is_last2_transpose(inner.args[1])
        if kn is None:
            continue
        vn = pv.args[1]
        kb, gk = _strip_kv_repeat(kn)
        vb, gv = _strip_kv_repeat(vn)
        if gk == gv and gk > 1:            # grouped-query attention written with repeated K / V
            kn, vn = kb, vb
        m = Match(qn, kn, vn, f1 * f2 * f3, mask_node is not None, pv, "explicit", gqa=(gk == gv and gk > 1))
        if mask_node is not None:
            _explicit_mask(gm, m, mask_node, how)
        found.append(m)
    return found


def _meta(n):
    tm = n.meta.get("tensor_meta") if isinstance(n, fx.Node) else None
    return tm


def legality(m: Match) -> str | None:
    """None when the fused kernel computes exactly this region, else the reason."""
    tq, tk, tv = _meta(m.q), _meta(m.k), _meta(m.v)
    if tq is None or tk is None or tv is None:
        return "no shape information"
    if m.error is not None:
        return m.error
    if len(tq.shape) != 4 or len(tk.shape) != 4 or len(tv.shape) != 4:
        return "operands are not [B, H, S, d]"
    if not (tq.dtype == tk.dtype == tv.dtype) or tq.dtype not in (torch.bfloat16, torch.float32):
        return f"dtype {tq.dtype} / {tk.dtype} / {tv.dtype} (bf16 or fp32, all alike)"
    B, Hq, Sq, d = tq.shape
    Bk, Hkv, Skv, dk = tk.shape
    if tuple(tv.shape) != (Bk, Hkv, Skv, tv.shape[3]) or tv.shape[3] != d or dk != d:
        return "K / V shapes"
    if d not in (64, 128):
        return f"head dim {d}"
    if Bk != B or Hq % Hkv != 0:
        return "batch or head counts"
    if Hq != Hkv and not (m.gqa or (m.kind == "explicit" and Hkv == 1)):
        return "query and KV head counts differ without grouping (enable_gqa, repeated K / V, or one KV head)"
    if m.causal and Sq > Skv:
        return "causal with more queries than keys (some rows would see no key)"
    return None


@dataclasses.dataclass
class Report:
    rewritten: list
    skipped: list


def rewrite(module: torch.nn.Module, *example_inputs) -> tuple[fx.GraphModule, Report]:
    """Trace ``module``, propagate shapes of ``example_inputs`` (on the meta
    device: no attention is computed), and replace every legal match by a call
    of :func:`fused_attention`.  Returns the rewritten GraphModule and a report
    of what was rewritten and what was skipped and why."""
    tracer = fx.Tracer()
    tracer.proxy_buffer_attributes = True     # buffers (e.g. a mask sliced by a traced length) become graph nodes
    graph = tracer.trace(module)
    gm = fx.GraphModule(tracer.root, graph)
    # shapes on a meta copy (parameters and buffers included), values of masks from the real attributes
    meta_gm = copy.deepcopy(gm).to("meta")
    _ShapeAndScalarProp(meta_gm).propagate(*[x.to("meta") if isinstance(x, torch.Tensor) else x
                                             for x in example_inputs])
    by_name = {n.name: n for n in meta_gm.graph.nodes}
    for n in gm.graph.nodes:
        n.meta.update(by_name[n.name].meta)
    rep = Report([], [])
    replaced = {}            # output node of a rewritten region -> its fused call
    for m in find_attention(gm):
        why = legality(m)
        if why is not None:
            rep.skipped.append((m.out.name, why))
            continue
        scale = m.scale if m.scale is not None else 1.0 / math.sqrt(_meta(m.q).shape[3])
        kw = {"causal": m.causal, "scale": scale}
        if m.causal and m.align != "top_left":
            kw["align"] = m.align
        if m.mask_lengths is not None:
            kw["lengths"] = m.mask_lengths
        # an input may be the output of a region rewritten just before (the
        # matches were all found on the original graph)
        q, k, v = (replaced.get(x, x) for x in (m.q, m.k, m.v))
        with gm.graph.inserting_after(m.out):
            fused = gm.graph.call_function(fused_attention, (q, k, v), kw)
        m.out.replace_all_uses_with(fused)
        replaced[m.out] = fused
        rep.rewritten.append((m.out.name, m.kind, m.causal, scale))
    gm.graph.eliminate_dead_code()
    gm.recompile()
    return gm, rep
