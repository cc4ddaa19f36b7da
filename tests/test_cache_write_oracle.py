"""Pins for the cache-write oracle: the slot scatter against numpy fancy indexing
on a slot-major view of the pool, an untouched-bytes check, padding slots, and
a planted mistake."""
import numpy as np
import pytest

import oracle


def _case(seed, NB=12, Hkv=3, BS=4, D=5, T=9):
    rng = np.random.default_rng(seed)
    kp = rng.integers(-2**15, 2**15, size=(NB, Hkv, BS, D), dtype=np.int16)
    vp = rng.integers(-2**15, 2**15, size=(NB, Hkv, BS, D), dtype=np.int16)
    kn = rng.integers(-2**15, 2**15, size=(T, Hkv, D), dtype=np.int16)
    vn = rng.integers(-2**15, 2**15, size=(T, Hkv, D), dtype=np.int16)
    slots = rng.choice(NB * BS, size=T, replace=False).astype(np.int32)
    slots[2] = -1
    return kp, vp, kn, vn, slots, BS


def _fancy(pool, new, slots, BS):
    """Same scatter through a [NB*BS, Hkv, D] slot-major view (a library route)."""
    NB, Hkv, _, D = pool.shape
    view = pool.transpose(0, 2, 1, 3).reshape(NB * BS, Hkv, D).copy()
    keep = slots >= 0
    view[slots[keep]] = new[keep]
    return view.reshape(NB, BS, Hkv, D).transpose(0, 2, 1, 3)


@pytest.mark.parametrize("seed", range(3))
def test_write_equals_fancy_index(seed):
    kp, vp, kn, vn, slots, BS = _case(seed)
    k2, v2 = oracle.kv_cache_write(kp, vp, kn, vn, slots, BS)
    assert np.array_equal(k2, _fancy(kp, kn, slots, BS))
    assert np.array_equal(v2, _fancy(vp, vn, slots, BS))


def test_untouched_bytes_and_padding():
    kp, vp, kn, vn, slots, BS = _case(5)
    k2, _ = oracle.kv_cache_write(kp, vp, kn, vn, slots, BS)
    touched = np.zeros(kp.shape[0] * BS, dtype=bool)
    touched[slots[slots >= 0]] = True
    touched = touched.reshape(kp.shape[0], BS)
    for b in range(kp.shape[0]):
        for o in range(BS):
            if not touched[b, o]:
                assert np.array_equal(k2[b, :, o], kp[b, :, o])
    # the padding token (slot -1) wrote nowhere
    assert not any(np.array_equal(k2[b, :, o], kn[2]) and not np.array_equal(kp[b, :, o], kn[2])
                   for b in range(kp.shape[0]) for o in range(BS) if not touched[b, o])
    # inputs are not modified in place
    kp0 = kp.copy()
    oracle.kv_cache_write(kp, vp, kn, vn, slots, BS)
    assert np.array_equal(kp, kp0)


def test_out_of_range_slot_rejected():
    kp, vp, kn, vn, slots, BS = _case(6)
    slots[0] = kp.shape[0] * BS
    with pytest.raises(ValueError):
        oracle.kv_cache_write(kp, vp, kn, vn, slots, BS)


WRITE_MUTANTS = {
    "block and offset swapped": ("block, offset = divmod(slot, block_size)",
                                 "offset, block = divmod(slot, block_size)"),
    "V written into K": ("k_out[block, :, offset, :] = k_new[t]", "k_out[block, :, offset, :] = v_new[t]"),
    "padding written": ("if slot < 0:\n            continue", "if slot < -1:\n            continue"),
    "token index shifted": ("v_out[block, :, offset, :] = v_new[t]",
                            "v_out[block, :, offset, :] = v_new[t - 1]"),
}


@pytest.mark.parametrize("name", sorted(WRITE_MUTANTS))
def test_planted_mistake_is_caught(name):
    import os
    import types
    from oracle import cache_write
    old, new = WRITE_MUTANTS[name]
    src = open(os.path.join(os.path.dirname(cache_write.__file__), "cache_write.py")).read()
    assert src.count(old) == 1
    mod = types.ModuleType("write_mutant")
    exec(compile(src.replace(old, new), "write_mutant", "exec"), mod.__dict__)
    caught = False
    for seed in range(3):
        kp, vp, kn, vn, slots, BS = _case(seed)
        try:
            k2, v2 = mod.kv_cache_write(kp, vp, kn, vn, slots, BS)
            ok = (np.array_equal(k2, _fancy(kp, kn, slots, BS))
                  and np.array_equal(v2, _fancy(vp, vn, slots, BS)))
        except Exception:
            ok = False
        caught |= not ok
    assert caught
