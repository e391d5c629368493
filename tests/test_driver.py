"""Host logic of the multi-layer driver: the anchor / reuse schedule (R35)."""
import pytest

from sparse_attention_diffusion_attn_amd.driver import LayerShape, Schedule


def test_schedule_kinds():
    assert Schedule(6, warmup=2, refresh=0).kinds() == ["dense", "anchor", "reuse", "reuse", "reuse", "reuse"]
    assert Schedule(8, warmup=3, refresh=3).kinds() == ["dense", "dense", "anchor", "reuse", "reuse",
                                                        "anchor", "reuse", "reuse"]
    assert Schedule(4, warmup=0, refresh=2).kinds() == ["anchor", "reuse", "anchor", "reuse"]
    assert Schedule(3, warmup=1, refresh=1).kinds() == ["anchor"] * 3
    with pytest.raises(ValueError):
        Schedule(0, 1, 1)


def test_entry_bytes():
    s = LayerShape(1, 24, 32760, 32768, 128, 128, 8190)
    assert s.entry_bytes() == 24 * (32768 * 4 + 256 * 8190 * 4 + 32768 * 128 * 2)
