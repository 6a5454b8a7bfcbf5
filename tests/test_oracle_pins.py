"""The CPU oracle agrees with every independent pin (see oracle_pins.py)."""
import pytest

import oracle
import oracle.paged_attention as opa
import oracle.block_manager as obm
import oracle.prefill as opr
from oracle_pins import ALL_PINS, BM_PINS, PREFILL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_oracle_pin(pin):
    pin(opa)


@pytest.mark.parametrize("pin", PREFILL_PINS, ids=[p.__name__ for p in PREFILL_PINS])
def test_prefill_oracle_pin(pin):
    pin(opr)


@pytest.mark.parametrize("pin", BM_PINS, ids=[p.__name__ for p in BM_PINS])
def test_block_manager_model_pin(pin):
    pin(obm)


def test_oracle_imports_only_numpy():
    """The oracle shares no code with the GPU path: it imports numpy only."""
    import ast
    import inspect

    for mod in (oracle, opa, opr):
        tree = ast.parse(inspect.getsource(mod))
        names = set()
        for node in ast.walk(tree):
            if isinstance(node, ast.Import):
                names.update(a.name.split(".")[0] for a in node.names)
            elif isinstance(node, ast.ImportFrom) and node.level == 0:
                names.add(node.module.split(".")[0])
        assert names <= {"numpy", "__future__"}, names
