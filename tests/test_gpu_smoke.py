"""The package's smoke check (`__graft_entry__.smoke`: one tiny forward + backward on cuda:0
against the oracle) as a GPU test, so that a change that breaks it fails the suite."""
import os
import sys

import pytest

from gpu_util import require_gpu

pytestmark = pytest.mark.gpu


def test_smoke_runs_green():
    require_gpu()
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import __graft_entry__
    __graft_entry__.smoke()
