"""The oracle against its pins (CPU only): worked cases, closed forms,
invariants, library routines and the pure-loop brute force."""
import zlib

import numpy as np
import pytest

from oracle import brute
from pins import ALL_CHECKS, oracle_ns


@pytest.mark.parametrize("name,check", ALL_CHECKS, ids=[n for n, _ in ALL_CHECKS])
def test_pin(name, check):
    check(oracle_ns(), brute, np.random.Generator(np.random.PCG64(zlib.crc32(name.encode()))))
