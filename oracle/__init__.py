"""CPU oracle for the int4-weight quantized linear layer -- TEST INFRASTRUCTURE.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import or call anything in this package. The product path (the HIP library
and its Python binding) never does, and shares no code with it.
"""
from .w4_oracle import *  # noqa: F401,F403
