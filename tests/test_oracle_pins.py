"""The fp64 oracle against its pins (CPU only)."""
import pytest

import oracle
from oracle_pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(oracle._load())


def test_rejects_out_of_domain():
    import numpy as np
    x = np.zeros((2, 8))
    for kw in (dict(K=0), dict(K=9), dict(K=4, num_groups=3, group_topk=1),
               dict(K=3, num_groups=4, group_topk=2),
               dict(K=4, num_groups=4, group_topk=5)):
        with pytest.raises(oracle.OracleError):
            oracle.topk_fwd(x, **kw)
    with pytest.raises(oracle.OracleError):
        oracle.topk_fwd(x, 2, oracle.SOFTMAX, bias=np.zeros(8))


def test_threads_split_matches_single():
    import numpy as np
    rng = np.random.default_rng(3)
    x = rng.normal(0, 1, (37, 40))
    b = rng.uniform(-.1, .1, 40)
    one = oracle.topk_fwd(x, 6, oracle.SIGMOID, True, 4, 2, 2.0, b,
                          threads=1)
    many = oracle.topk_fwd(x, 6, oracle.SIGMOID, True, 4, 2, 2.0, b,
                           threads=5)
    for u, v in zip(one, many):
        assert (u == v).all()
