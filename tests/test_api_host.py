"""Host logic of the one-call API (no GPU): the scale block it asks the
quantiser for on the dense and sliding-tile paths, and which operand copies
it requests."""
from precision_attention_block_amd import api


class _Plan:
    tile_tokens, perm, n_tokens = 384, None, 46080


def _record(monkeypatch):
    seen = []

    def quantize(x, recipe, block_tokens=None, perm=None, n_out=None, operand=True):
        seen.append((x, recipe, block_tokens, operand))
        return recipe

    monkeypatch.setattr(api.B, "quantize", quantize)
    monkeypatch.setattr(api.B, "attention_sta", lambda *a, **k: "out")
    monkeypatch.setattr(api.B, "attention_dense", lambda *a, **k: "out")
    return seen


def test_sta_default_scale_block_is_one_tile(monkeypatch):
    """Without block_tokens the sliding-tile path quantises Q and K with one
    FP8 scale per 3D tile (FPSAttention page, §2.3 and §3.1)."""
    seen = _record(monkeypatch)
    api.attention("q", "k", "v", recipe="fp8", sta=_Plan())
    assert [(r, b) for _, r, b, _ in seen[:2]] == [("fp8_block", 384)] * 2
    seen.clear()
    api.attention("q", "k", "v", recipe="fp8", sta=_Plan(), block_tokens=128)
    assert [b for _, _, b, _ in seen[:2]] == [128, 128]


def test_dense_default_scale_block(monkeypatch):
    seen = _record(monkeypatch)
    api.attention("q", "k", "v", recipe="fp8")
    assert [(r, b) for _, r, b, _ in seen[:2]] == [("fp8_block", 128)] * 2


def test_forward_skips_q_operand_copy(monkeypatch):
    """The forward needs K's bf16 operand copy only; the training path keeps
    Q's too, for the backward."""
    seen = _record(monkeypatch)
    api.quantize_qkv("q", "k", "v", "fp8", 64)
    ops = {x: op for x, _, _, op in seen}
    assert ops["q"] is False and ops["k"] is True
    seen.clear()
    api.quantize_qkv("q", "k", "v", "fp8", 64, q_operand=True)
    assert {x: op for x, _, _, op in seen}["q"] is True
