"""CPU oracle for the tile quantizer and its paged decode-attention read path.

Test infrastructure only: the tests, the smoke check and the bench's CPU
baseline may import it; the product path never does.  See kvq_oracle.py.
"""
from .kvq_oracle import *  # noqa: F401,F403
