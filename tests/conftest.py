import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: takes more than a few seconds")


_WEIGHTS = {}


@pytest.fixture(scope="session")
def weights_cache():
    """Seeded weights are expensive at full width: share them per session."""
    import synth

    def get(name):
        if name not in _WEIGHTS:
            _WEIGHTS[name] = synth.make_weights(synth.model_config(name))
        return _WEIGHTS[name]
    return get
