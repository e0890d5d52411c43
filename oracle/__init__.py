"""CPU float64 oracle for the KATA causal forward.

Test infrastructure only: the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import it; the library path never does.
"""
from .kata_oracle import *  # noqa: F401,F403
from .first_order_oracle import *  # noqa: F401,F403
from .decay_oracle import *  # noqa: F401,F403
from .delta_oracle import *  # noqa: F401,F403
from .factored_oracle import *  # noqa: F401,F403
