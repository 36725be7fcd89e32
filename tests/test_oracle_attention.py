"""Pins of the oracle's attention against a library routine and closed forms,
for both of its forms: the numpy one and the C one (attention.c, OpenMP).
CPU only."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import tracegen as tg
from oracle import attention as oatt


def _tiny(latent=False, tpe=1, Hkv=2, G=4, dqk=16, dv=16, N=40, k=7, T=2, batch=2):
    return tg.WORKLOADS[1].replace(batch=batch, n_kv_heads=Hkv, n_q_heads=Hkv * G, n_q_tokens=T,
                                   head_dim_qk=dqk, head_dim_v=dv if not latent else dv,
                                   latent=latent, n_entries=N, tokens_per_entry=tpe, k=k,
                                   n_slots=2 * T * k)


IMPLS = ["numpy", "c"]


def _attend(impl, w, q, host, sel, lengths=None):
    if impl == "numpy":
        return oatt.attend(w, q, host, sel, lengths=lengths)
    return oatt.attend_native(w, q, np.ascontiguousarray(host), sel, lengths=lengths, threads=3)


def _bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits by truncation (test data only)."""
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("impl", IMPLS)
@pytest.mark.parametrize("layout", ["token", "page", "latent"])
def test_matches_masked_sdpa(layout, impl):
    """Attention over the selected set equals torch's scaled_dot_product_attention
    over ALL positions with a boolean mask that keeps the selected ones, with
    torch's own grouped-query head mapping (enable_gqa)."""
    if layout == "latent":
        w = _tiny(latent=True, Hkv=1, G=8, dqk=24, dv=16)
    elif layout == "page":
        w = _tiny(tpe=4)
    else:
        w = _tiny()
    rng = np.random.default_rng(7)
    host = _bits(rng.standard_normal((w.units, w.n_entries, w.row_elems)))
    q = _bits(rng.standard_normal((w.batch, w.n_q_tokens, w.n_q_heads, w.head_dim_qk)))
    sel = np.stack([np.stack([np.sort(rng.choice(w.n_entries, w.k, replace=False))
                              for _ in range(w.n_q_tokens)]) for _ in range(w.units)]).astype(np.int32)
    out = _attend(impl, w, q, host, sel)

    # dense K/V over every position of every unit, token-major
    tpe = w.tokens_per_entry
    hk = oatt.bf16_to_f64(host)                                   # [units][N][row]
    if w.latent:
        Kd, Vd = hk[..., :w.head_dim_qk], hk[..., :w.head_dim_v]
    else:
        Kd = hk[..., :tpe * w.head_dim_qk].reshape(w.units, w.n_entries * tpe, w.head_dim_qk)
        Vd = hk[..., tpe * w.head_dim_qk:].reshape(w.units, w.n_entries * tpe, w.head_dim_v)
    Kd = torch.from_numpy(Kd).reshape(w.batch, w.n_kv_heads, -1, w.head_dim_qk)
    Vd = torch.from_numpy(Vd).reshape(w.batch, w.n_kv_heads, -1, w.head_dim_v)
    for j in range(w.n_q_tokens):
        Q = torch.from_numpy(oatt.bf16_to_f64(q[:, j]))[:, :, None, :]     # [B][Hq][1][d]
        mask = torch.zeros(w.batch, w.n_q_heads, 1, w.n_entries * tpe, dtype=torch.bool)
        G = w.n_q_heads // w.n_kv_heads
        for u in range(w.units):
            b, g = divmod(u, w.n_kv_heads)
            pos = (sel[u, j][:, None] * tpe + np.arange(tpe)[None, :]).ravel()
            mask[b, g * G:(g + 1) * G, 0, torch.from_numpy(pos)] = True
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q, Kd, Vd, attn_mask=mask, scale=w.softmax_scale, enable_gqa=True)
        np.testing.assert_allclose(out[:, j], ref[:, :, 0].numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("impl", IMPLS)
def test_equal_keys_give_mean_of_values(impl):
    """All selected keys equal => uniform weights => o = mean of the values."""
    w = _tiny(T=1, batch=1, Hkv=1)
    rng = np.random.default_rng(3)
    host = _bits(rng.standard_normal((1, w.n_entries, w.row_elems)))
    host[0, :, :w.head_dim_qk] = host[0, 0, :w.head_dim_qk]
    q = _bits(rng.standard_normal((1, 1, w.n_q_heads, w.head_dim_qk)))
    sel = np.sort(rng.choice(w.n_entries, w.k, replace=False)).astype(np.int32)[None, None]
    out = _attend(impl, w, q, host, sel)
    V = oatt.bf16_to_f64(host[0, sel[0, 0], w.head_dim_qk:])
    np.testing.assert_allclose(out[0, 0], np.broadcast_to(V.mean(0), out[0, 0].shape), atol=1e-12)


@pytest.mark.parametrize("impl", IMPLS)
def test_single_entry_returns_its_value(impl):
    w = _tiny(T=1, batch=1, Hkv=1, k=1)
    rng = np.random.default_rng(4)
    host = _bits(rng.standard_normal((1, w.n_entries, w.row_elems)))
    q = _bits(rng.standard_normal((1, 1, w.n_q_heads, w.head_dim_qk)))
    sel = np.array([[[11]]], np.int32)
    out = _attend(impl, w, q, host, sel)
    V = oatt.bf16_to_f64(host[0, 11, w.head_dim_qk:])
    np.testing.assert_allclose(out[0, 0], np.broadcast_to(V, out[0, 0].shape), atol=0)


@pytest.mark.parametrize("impl", IMPLS)
def test_one_dominant_key(impl):
    """A key far more aligned with q than the others takes all the weight."""
    w = _tiny(T=1, batch=1, Hkv=1, G=1)
    host = np.zeros((1, w.n_entries, w.row_elems), np.float32)
    host[0, :, w.head_dim_qk:] = np.arange(w.n_entries)[:, None]
    host[0, 9, :w.head_dim_qk] = 8.0
    q = np.full((1, 1, 1, w.head_dim_qk), 8.0, np.float32)
    sel = np.array([[[2, 5, 9, 20, 30, 31, 39]]], np.int32)
    out = _attend(impl, w, _bits(q), _bits(host), sel)
    np.testing.assert_allclose(out[0, 0, 0], 9.0, atol=1e-9)


@pytest.mark.parametrize("impl", IMPLS)
def test_lengths_attend_over_the_prefix_only(impl):
    """With per-list lengths, attention equals masked SDPA over the first len
    entries; what follows them (here ids of other entries) plays no part."""
    w = _tiny(T=1)
    rng = np.random.default_rng(9)
    host = _bits(rng.standard_normal((w.units, w.n_entries, w.row_elems)))
    q = _bits(rng.standard_normal((w.batch, 1, w.n_q_heads, w.head_dim_qk)))
    sel = np.stack([np.sort(rng.choice(w.n_entries, w.k, replace=False))[None]
                    for _ in range(w.units)]).astype(np.int32)
    lens = rng.integers(1, w.k + 1, size=(w.units, 1)).astype(np.int32)
    got = _attend(impl, w, q, host, sel, lengths=lens)
    hk = oatt.bf16_to_f64(host)
    G = w.n_q_heads // w.n_kv_heads
    for u in range(w.units):
        b, g = divmod(u, w.n_kv_heads)
        mask = torch.zeros(w.n_entries, dtype=torch.bool)
        mask[torch.from_numpy(sel[u, 0, :lens[u, 0]].astype(np.int64))] = True
        qq = torch.from_numpy(oatt.bf16_to_f64(q[b, 0, g * G:(g + 1) * G]))[None, :, None, :]
        K = torch.from_numpy(hk[u, :, :w.head_dim_qk])[None, None]
        V = torch.from_numpy(hk[u, :, w.head_dim_qk:])[None, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qq, K.expand(1, G, -1, -1), V.expand(1, G, -1, -1), attn_mask=mask[None, None, None, :],
            scale=w.softmax_scale)[0, :, 0, :].numpy()
        assert np.allclose(got[b, 0, g * G:(g + 1) * G], ref, rtol=1e-10, atol=1e-12)


def test_native_threads_and_failed_units():
    """The C attention gives the same bits on 1 and on 5 threads (each (unit,
    token, head) is computed by one thread, in selection order), and a unit
    whose step failed yields zeros."""
    w = _tiny(tpe=2)
    rng = np.random.default_rng(11)
    host = _bits(rng.standard_normal((w.units, w.n_entries, w.row_elems)))
    q = _bits(rng.standard_normal((w.batch, w.n_q_tokens, w.n_q_heads, w.head_dim_qk)))
    sel = np.stack([np.stack([np.sort(rng.choice(w.n_entries, w.k, replace=False))
                              for _ in range(w.n_q_tokens)]) for _ in range(w.units)]).astype(np.int32)
    status = np.zeros(w.units, np.int32)
    status[1] = 17
    a = oatt.attend_native(w, q, host, sel, status, threads=1)
    b = oatt.attend_native(w, q, host, sel, status, threads=5)
    assert np.array_equal(a, b)
    G = w.n_q_heads // w.n_kv_heads
    assert (a[0, :, G:2 * G] == 0).all()   # unit 1 = request 0, KV head 1
    np.testing.assert_allclose(a, oatt.attend(w, q, host, sel, status), rtol=1e-12, atol=1e-13)
