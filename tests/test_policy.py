"""Per-layer policy (selective layer skipping, summary page, method step 3) and the layer
object's host-side checks.  CPU only."""
import pytest

from activation_sparse_gemm_amd import policy


def test_skip_lists_follow_the_page():
    # Qwen-Image (double stream): QKV, MLP up and MLP down are sparsified
    for kind in ("attn.qkv", "mlp.up", "mlp.down"):
        assert policy.is_sparse("qwen-image", "double", kind)
    # FLUX single-stream path keeps attn.o_proj and mlp.down dense; the rest is sparse
    assert not policy.is_sparse("flux", "single", "attn.o_proj")
    assert not policy.is_sparse("flux", "single", "mlp.down")
    assert policy.is_sparse("flux", "single", "attn.qkv")
    assert policy.is_sparse("flux", "single", "mlp.up")
    # Z-Image keeps attn.o_proj and mlp.up dense
    assert not policy.is_sparse("z-image", "single", "attn.o_proj")
    assert not policy.is_sparse("z-image", "single", "mlp.up")
    assert policy.is_sparse("z-image", "single", "attn.qkv")
    assert policy.is_sparse("z-image", "single", "mlp.down")


def test_readings_where_the_page_is_silent():
    assert not policy.is_sparse("qwen-image", "double", "attn.o_proj")
    assert all(policy.is_sparse("flux", "double", k) for k in policy.LAYER_KINDS)


def test_unknown_names_raise():
    with pytest.raises(KeyError):
        policy.is_sparse("sd3", "double", "attn.qkv")
    with pytest.raises(KeyError):
        policy.is_sparse("flux", "single", "attn.q")
    with pytest.raises(KeyError):
        policy.dense_layers("z-image", "double")


def test_case_insensitive_and_models_listed():
    assert policy.dense_layers("FLUX", "Single") == policy.dense_layers("flux", "single")
    assert set(policy.MODELS) == {"flux", "qwen-image", "z-image"}


def test_linear_requires_both_factors():
    import torch
    W = torch.zeros((4, 8))
    with pytest.raises(ValueError):
        policy.Linear(W, LA=torch.zeros((4, 2)), LB=None)
    assert policy.Linear(W, sparse=False).R == 0
